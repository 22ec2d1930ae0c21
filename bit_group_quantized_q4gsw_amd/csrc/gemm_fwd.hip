// MFMA forward for M > 8:  y[m, n] = sum_k x[m, k] * (code[n, k] - 8) * scale[k / gs, n].
//
// The forward GEMM of the pages (the linear_q4gsw op; the WebGPU BK64 QKV PR body
// mirrors the Vulkan q4gsw forward GEMM per projection) re-designed for gfx950:
//
//   * v_mfma_f32_32x32x16 with fp32 accumulators; a wave owns a 32 MI (M) x 32 (N) output
//     tile = MI MFMA tiles (MI = 4, or 2 for short activations), so every dequantised code
//     feeds 32 MI activation rows;
//   * block = 8 waves side by side in N (block tile 32 MI x 256), two waves per SIMD, so the
//     code unpacking of one wave issues while the other wave's MFMAs run;
//   * every global read is an LDS-DMA (global_load_lds): the activation chunk (64 columns;
//     128 in the exact-code group mode with gs == 128, so every chunk opens one group and the
//     chunk loop is one straight-line path) shared by the 8
//     waves, each wave's 1 or 2 KB of codes and its scales travel straight
//     into a ring of KD + 1 LDS stages, KD chunks ahead of the MFMAs, with no VGPR
//     staging.  Explicit vmcnt waits + s_barrier order the ring; the compiler only sees
//     LDS reads (fp32 activations are the exception: split into bf16 hi + lo planes in
//     registers on their way into LDS);
//   * LDS swizzles: activation k-octet slots of row r sit at slot (octet ^ ((r >> 1) & 7))
//     for 128-byte rows and (octet ^ (r & 15)) for 256-byte rows, so the 16 lanes of an
//     A-fragment read phase (16 rows) cover all 64 banks; each 256-byte code run of
//     row-octet R is rotated by 2R 32-byte blocks, so the 64 lanes reading one k-octet pair
//     of the wave's 4 row-octets hit 64 distinct banks;
//   * the K range is split across blocks when the output tiles cannot fill the GPU; the
//     split index is the fastest-varying block coordinate, so with 8 splits every XCD owns
//     one K slice (its activation and code slices stay in that XCD's L2); a reduction
//     kernel sums the split partials.
//
// K order inside a chunk: MFMA step t contracts k-octets 2t (lanes 0..31) and 2t+1 (lanes
// 32..63), so a step covers 16 consecutive columns.
//
// Precision routes (all with fp32 accumulation):
//   kModeFold  (fp16 x, fp16 scales checked foldable at pack time):
//       B = fp16((code - 8) * scale), one rounding, |err| <= 2^-11 |w|.
//   kModeGroup (fp16 or bf16 x): B = code - 8 held exactly (fp16, or bf16 of (code - 8) / 16)
//       and the scale multiplies the fp32 partial sum of each scale group, which the MFMAs
//       build in a separate set of accumulators.
//   kModeSplit (fp32 x): x = hi + lo in bf16 (|err| <= 2^-18 |x|), two MFMA passes
//       against the exact bf16 codes, scale per group as in kModeGroup.
#include "device.h"
#include "internal.h"

#include <atomic>
#include <type_traits>

namespace q4gsw {

constexpr int kWaves = 8;           // waves per block, two per SIMD
constexpr int kWN = 32;             // wave columns (N)
constexpr int kBN = kWaves * kWN;   // block columns (N)
constexpr int kCK = 64;             // K columns per chunk (kCKWide in the wide group instances)
constexpr int kCKWide = 128;
#ifndef Q4GSW_FWD_DEPTH
#define Q4GSW_FWD_DEPTH 2
#endif
constexpr int kDepth16 = Q4GSW_FWD_DEPTH;   // chunks in flight ahead of the one multiplied (16-bit x)

struct FwdSegArgs {
    const uint8_t* nib[3];
    const void* scales[3];
    float* out[3];                // final output (splits == 1) or the workspace
    int64_t N[3];
    int64_t n_pad[3];
    int64_t out_ld[3];            // row pitch of out (splits == 1)
    int64_t col0[3];              // splits > 1: first workspace column of the segment
    int64_t ntn;                  // splits > 1: 32-column tiles across the workspace
    int64_t tile_start[4];        // first N tile of each segment (prefix sums), tile_start[nseg] = total
    int64_t g_pad;                // scale groups stored (shared: the segments share K and group size)
    int nseg;
    // XCD-aware block order (blocks b and b + 8 run on one XCD): xcd_g = 8 / splits XCDs share a
    // split; each takes a contiguous 1/xcd_g of the (column tile, row tile) pairs, column tiles
    // outermost when xcd_cols (the weight is split across XCDs and the activation repeated), else
    // row tiles.  xcd_g = 1: row tile, then column tile, after the split index.
    int xcd_g;
    int xcd_cols;
    // low-rank term of a one-split, one-segment launch (P == nullptr: none): y += alpha t G^T with
    // G = lr.G [N, rank] and t from its column-chunk partials, as the adapter's expansion does it
    LowRankEpi lr;
};

// bf16 pair ((c_lo - 8) / 16, (c_hi - 8) / 16) of dword e of a code word's MFMA fragment: nibble
// positions e (low half) and e + 4 (high half).  With X = w ^ 0x88888888 (every nibble the
// two's-complement 4-bit c - 8) and Xs = X >> 4, position 2b sits in the low nibble of byte b of
// X and position 2b + 1 in the low nibble of byte b of Xs.  v_cvt_off_f32_i4 reads the low
// nibble of a byte select (SDWA) and gives (c - 8) / 16 exactly; its upper half is the exact
// bf16.  Seven VALU per two codes fewer than widening signed bytes: no masks per word.
__device__ __forceinline__ uint32_t code_pair_bf16(uint32_t X, uint32_t Xs, int e) {
    const uint32_t src = (e & 1) ? Xs : X;
    const int by = e >> 1;
    const float lo = __builtin_amdgcn_cvt_off_f32_i4((int)((src >> (8 * by)) & 0xFFu));
    const float hi = __builtin_amdgcn_cvt_off_f32_i4((int)((src >> (8 * (by + 2))) & 0xFFu));
    return __builtin_amdgcn_perm(bitcast<uint32_t>(hi), bitcast<uint32_t>(lo), 0x07060302u);
}

// SPC: scale slots per chunk (1: gs % 64 == 0; 2: gs % 32 == 0, one slot per 32 columns, which
// the group and split modes take only for gs == 32; 4: fold mode with any gs % 8 == 0, one slot
// per k-octet of the lane).  SF: 1 = fp16 scales.
// Wait until at most n (clamped to 0..N) chunks of PER loads each issued after the chunk about
// to be read are outstanding, then meet the other waves.
template <int PER, int N>
__device__ __forceinline__ void wait_chunks_barrier(int64_t n) {
    if constexpr (N == 0) {
        wait_loads_barrier<0>();
    } else {
        if (n >= N) wait_loads_barrier<N * PER>();
        else wait_chunks_barrier<PER, N - 1>(n);
    }
}

// LDS slot swizzle of activation row r: 128-byte rows (64 columns) pair rows across the two
// 32-bank halves, 256-byte rows (128 columns) give 16 rows 16 distinct slots.
template <int CW>
__device__ __forceinline__ int a_swizzle(int r) {
    if constexpr (CW == kCK) return (r >> 1) & 7;
    else return r & 15;
}

// RG: the activation may be ragged (K % CW != 0) or not 16-byte aligned, so chunks can take the
// synchronous fallback; the aligned instance carries no fallback code (and none of its live
// values across the chunk loop).  CW: K columns per chunk, 64, or 128 for the exact-code group
// mode with gs == 128.  LR: the one-split epilogue adds the low-rank term seg.lr.
template <int XT, int MODE, int SPC, int SF, int MI, int KD, bool RG, int CW, bool LR = false>
__global__ __launch_bounds__(512, 1) void gemm_fwd_kernel(FwdSegArgs seg, const void* __restrict__ x, int64_t M,
                                                          int64_t K, int64_t k_pad, int64_t gs, int x_fast,
                                                          int chunks_per_split, int splits, int mtiles,
                                                          int64_t split_stride) {
    static_assert(MI == 2 || MI == 4, "32-row MFMA tiles per wave");
    static_assert(KD >= 2 && KD <= 6 && (XT != kF32 || KD == 2), "chunks in flight");
    static_assert(CW == kCK || (CW == kCKWide && XT != kF32 &&
                                ((MODE == kModeGroup && SPC == 1) || (MODE == kModeFold && SF == 1))),
                  "128-column chunks: exact-code group mode with one group per chunk (gs == 128), or fold mode");
    constexpr int kSteps = CW / 16;                       // MFMA steps per chunk
    constexpr int kRowBytes = 2 * CW;                     // one activation row (or bf16 plane row) of a chunk
    constexpr int kSlots = CW / 8;                        // 16-byte k-octet slots per row
    constexpr int kCodeBytes = 16 * CW;                   // one wave's codes of a chunk: 32 rows x CW x 4 bits
    constexpr int kCDma = CW / 64;                        // 1 KB code DMAs per wave per chunk
    constexpr int kStages = KD + 1;                       // LDS stages in the ring
    constexpr int kBM = 32 * MI;                          // block rows (M)
    constexpr int kRowsPerWave = kBM / kWaves;            // activation rows each wave stages
    constexpr int kPlaneBytes = kBM * kRowBytes;
    constexpr int kAUnits = kBM * 16 / (64 * kWaves);     // fp32 float4 units per thread per chunk
    constexpr bool kX16 = XT != kF32;
    constexpr int kPlanes = kX16 ? 1 : 2;
    constexpr int kRowsPerDma = 1024 / kRowBytes;         // activation rows of one 16-bit DMA
    constexpr int kADma = kX16 ? kRowsPerWave / kRowsPerDma : 0;   // activation DMAs per wave per chunk
    // Scales: a slot covers kSlotCols columns (SPC slots per chunk).  With slots of 32 columns or
    // more (SPC <= 2, or any SPC in 128-column chunks) wave 0 fetches the block's 256 rows in
    // kSDma0 16-byte-per-lane DMAs; with a slot per 16 columns (SPC == 4 in 64-column chunks)
    // every wave fetches its own rows, 4 bytes per lane.
    constexpr int kSlotCols = CW / SPC;
    constexpr bool kBlockScales = kSlotCols >= 32;
    constexpr int kSDma0 = SF ? (SPC > 2 ? SPC / 2 : 1) : SPC;   // block scale DMAs of wave 0 per chunk
    constexpr int kSDma = kBlockScales ? 0 : SPC;         // scale DMAs of every wave per chunk
    constexpr int kDmaPerChunk = kADma + kCDma + kSDma;
    constexpr int kDmaPerChunk0 = kDmaPerChunk + (kBlockScales ? kSDma0 : 0);   // wave 0
    constexpr int kAOff = 0;
    constexpr int kBOff = kPlanes * kPlaneBytes;
    constexpr int kSOff = kBOff + kWaves * kCodeBytes;
    constexpr int kStageBytes = kSOff + (kBlockScales ? 1024 * kSDma0 : kWaves * SPC * 256);
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: its address math stays scalar
    const int j = lane & 31;          // MFMA row / column inside a 32x32 tile
    const int h = lane >> 5;          // MFMA k-group: k-octet 2t + h of step t

    // ---- block -> (K split, M tile, N tile); the split index varies fastest ----
    const int64_t bid = blockIdx.x;
    const int z = (int)(bid % splits);
    const int64_t rest = bid / splits;
    int64_t mb, tile;
    if (seg.xcd_g > 1) {
        const int64_t ntiles = seg.tile_start[seg.nseg];
        const int64_t idx = (rest % seg.xcd_g) * (ntiles * mtiles / seg.xcd_g) + rest / seg.xcd_g;
        mb = seg.xcd_cols ? idx % mtiles : idx / ntiles;
        tile = seg.xcd_cols ? idx / mtiles : idx % ntiles;
    } else {
        mb = rest % mtiles;
        tile = rest / mtiles;
    }
    int sg = 0;
    while (sg + 1 < seg.nseg && tile >= seg.tile_start[sg + 1]) ++sg;
    const int64_t n0 = (tile - seg.tile_start[sg]) * kBN + (int64_t)wave * kWN;   // first W row of the wave
    const bool wave_active = n0 < seg.n_pad[sg];
    const int64_t nw = wave_active ? n0 : 0;   // an idle wave streams valid rows it never uses
    const int64_t m0 = mb * kBM;
    const int64_t kocts = k_pad >> 3;
    const int64_t n_chunks = (K + CW - 1) / CW;
    const int64_t c_begin = (int64_t)z * chunks_per_split;
    const int64_t c_end = min(c_begin + (int64_t)chunks_per_split, n_chunks);

    lds_u8* const sm_l = (lds_u8*)smem;

    // ---------------- DMA source addresses ----------------
    // Codes: one DMA per wave and 64 chunk columns covers the wave's 4 row-octets; lane l fills
    // LDS bytes 16 l = row-octet R = l >> 4, rotated block slot p = (l & 15) >> 1, half l & 1,
    // which holds k-octet (p - 2R) & 7 of those 64 columns.
    const uint8_t* csrc;
    {
        const int R = lane >> 4;
        const int p = (lane & 15) >> 1;
        const int o = (p - 2 * R) & 7;
        csrc = seg.nib[sg] + 32 * (((nw >> 3) + R) * kocts + o) + 16 * (lane & 1);
    }
    // Scales, per-wave form (SPC == 4): DMA lane (jj, hh) = (l & 31, l >> 5) loads, for k-group
    // hh, the fp32 scale of W row nw + jj or the fp16 pair of rows nw + 2 (jj & 15), +1
    // (adjacent in the scale plane).  Block form: row-octets boct .. boct + 31 of the tile.
    const int64_t srow = SF ? nw + 2 * (j & 15) : nw + j;
    const int64_t sbase = (srow >> 3) * (seg.g_pad * 8) + (srow & 7);
    const uint8_t* sptr = static_cast<const uint8_t*>(seg.scales[sg]);
    const int64_t boct = (tile - seg.tile_start[sg]) * (kBN / 8);
    const int64_t n_octs = seg.n_pad[sg] / 8;
    // Activations (16-bit): DMA q of wave w covers rows kRowsPerWave w + kRowsPerDma q onwards;
    // lane i fills slot i % kSlots of row i / kSlots, which holds k-octet slot ^ swz(row).
    const uint16_t* xa[kADma > 0 ? kADma : 1];
    int xoct[kADma > 0 ? kADma : 1];
    if constexpr (kX16) {
#pragma unroll
        for (int q = 0; q < kADma; ++q) {
            const int row = kRowsPerWave * wave + kRowsPerDma * q + lane / kSlots;
            xoct[q] = (lane % kSlots) ^ a_swizzle<CW>(row);
            const int64_t m = min(m0 + row, M - 1);     // rows past M only feed discarded outputs
            xa[q] = static_cast<const uint16_t*>(x) + m * K + 8 * xoct[q];
        }
    }

    auto issue_codes_scales = [&](int64_t c, int st) {
        lds_u8* base = sm_l + st * kStageBytes;
#pragma unroll
        for (int d = 0; d < kCDma; ++d) dma16(csrc + 256 * (kCDma * c + d), base + kBOff + wave * kCodeBytes + 1024 * d);
        const uint32_t kc = (uint32_t)(c * CW);
        const uint32_t ug = (uint32_t)gs;
        if constexpr (kBlockScales) {
            if (wave == 0) {
#pragma unroll
                for (int i = 0; i < kSDma0; ++i) {
                    // lane -> (row-octet o of the block, slot q, 16-byte half of an fp32 run);
                    // fp16 with SPC == 1: lanes 32..63 repeat lanes 0..31
                    int o, q, half;
                    if constexpr (SF) {
                        const int P = 64 * i + lane;
                        o = (P / SPC) & 31;
                        q = P % SPC;
                        half = 0;
                    } else {
                        const int P = 32 * i + (lane >> 1);
                        o = P / SPC;
                        q = P % SPC;
                        half = lane & 1;
                    }
                    const int64_t g = (int64_t)((kc + (uint32_t)kSlotCols * (uint32_t)q) / ug);
                    const int64_t oct = min(boct + o, n_octs - 1);   // rows past n_pad: a valid octet
                    const int64_t idx = (oct * seg.g_pad + g) * 8;
                    const uint8_t* src = SF ? sptr + 2 * idx : sptr + 4 * idx + 16 * half;
                    dma16(src, base + kSOff + 1024 * i);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < SPC; ++q) {
                const uint32_t k = kc + 16 * q + 8 * h;
                const int64_t idx = sbase + (int64_t)(k / ug) * 8;
                lds_u8* sdst = base + kSOff + wave * (SPC * 256) + 256 * q;
                if constexpr (SF) dma4(sptr + 2 * idx, sdst);
                else dma4(sptr + 4 * idx, sdst);
            }
        }
    };
    // Synchronous fallback for a ragged K tail or unaligned x: zero-filled register loads
    // into the slots the DMA would write.
    auto fill_a16_slow = [&](int64_t kc, int st) {
#pragma unroll
        for (int q = 0; q < kADma; ++q) {
            const int row = kRowsPerWave * wave + kRowsPerDma * q + lane / kSlots;
            const int64_t m = m0 + row;
            const int64_t k = kc + 8 * xoct[q];
            uint32_t e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                e[i] = (m < M && k + i < K) ? static_cast<const uint16_t*>(x)[m * K + k + i] : 0u;
            *reinterpret_cast<u4*>(smem + st * kStageBytes + kAOff + row * kRowBytes + 16 * (lane % kSlots)) =
                u4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
        }
    };
    auto issue_a16 = [&](int64_t c, int st) {
        const int64_t kc = c * CW;
        if (!RG || (x_fast && kc + CW <= K)) {
#pragma unroll
            for (int q = 0; q < kADma; ++q)
                dma16(xa[q] + kc, sm_l + st * kStageBytes + kAOff + (kRowsPerWave * wave + kRowsPerDma * q) * kRowBytes);
        } else if constexpr (RG) {
            fill_a16_slow(kc, st);
        }
    };

    // fp32 activations: kAUnits float4 units per thread, split into bf16 hi / lo planes at store time.
    f4 areg[kAUnits];
    auto load_a32 = [&](int64_t c) {
        const int64_t kc = c * CW;
        const bool fast = !RG || (x_fast && kc + CW <= K);
#pragma unroll
        for (int i = 0; i < kAUnits; ++i) {
            const int unit = tid + 64 * kWaves * i;
            const int row = unit >> 4;
            const int64_t k = kc + 4 * (unit & 15);
            if (fast) {
                const int64_t m = min(m0 + row, M - 1);
                areg[i] = *reinterpret_cast<const f4*>(static_cast<const float*>(x) + m * K + k);
            } else {
                const int64_t m = m0 + row;
                f4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = (m < M && k + e < K) ? static_cast<const float*>(x)[m * K + k + e] : 0.f;
                areg[i] = v;
            }
        }
    };
    auto store_a32 = [&](int st) {
#pragma unroll
        for (int i = 0; i < kAUnits; ++i) {
            const int unit = tid + 64 * kWaves * i;
            const int row = unit >> 4;
            const int oct = (unit & 15) >> 1;
            const int off = st * kStageBytes + kAOff + row * kRowBytes + 16 * (oct ^ ((row >> 1) & 7)) + 8 * (unit & 1);
            uint32_t h0, l0, h1, l1;
            split_bf16(areg[i].x, areg[i].y, h0, l0);
            split_bf16(areg[i].z, areg[i].w, h1, l1);
            *reinterpret_cast<u2*>(smem + off) = u2{h0, h1};
            *reinterpret_cast<u2*>(smem + kPlaneBytes + off) = u2{l0, l1};
        }
    };

    // ---------------- accumulators ----------------
    constexpr bool kGroup = MODE != kModeFold;
    f32x16 acc[MI];
    f32x16 part[kGroup ? MI : 1];            // partial sums of the open scale group
    float gopen = 0.f;                       // its scale (row n0 + j)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // ---------------- one chunk of MFMAs ----------------
    const int swz = a_swizzle<CW>(j);   // the swizzle of every A row (32 mi + j) this lane reads
    const int Rj = j >> 3;            // this lane's row-octet inside the wave
    // LDS byte of this lane's scale (row r = 32 wave + j) in slot q: block form, run
    // SPC (r >> 3) + q of 8 scales; per-wave form, half of a pair word (fp16) or a word (fp32)
    const int srl = 32 * wave + j;
    auto soff = [&](int q) -> int {
        if constexpr (kBlockScales) return (SF ? 16 : 32) * (SPC * (srl >> 3) + q) + (SF ? 2 : 4) * (srl & 7);
        else return 256 * q + (SF ? 4 * (32 * h + (j >> 1)) + 2 * (j & 1) : 4 * (32 * h + j));
    };
    // fp32 group scale of slot q for row n0 + j; bf16 codes carry a factor 1/16 that the scale
    // removes exactly.
    auto group_scale = [&](const uint8_t* S, int q) -> float {
        constexpr float kUnit = (XT == kF16) ? 1.0f : 16.0f;
        if constexpr (SF) return (float)bitcast<_Float16>(*reinterpret_cast<const uint16_t*>(S + soff(q))) * kUnit;
        else return *reinterpret_cast<const float*>(S + soff(q)) * kUnit;
    };
    // A fragments of step t for the wave's MI 32-row tiles (and the lo plane for fp32 x).
    auto read_a = [&](const uint8_t* Ab, int t, u4 (&a)[MI], u4 (&alo)[MI]) {
        const int slot = 16 * ((2 * t + h) ^ swz);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int off = (32 * mi + j) * kRowBytes + slot;
            a[mi] = *reinterpret_cast<const u4*>(Ab + off);
            if constexpr (MODE == kModeSplit) alo[mi] = *reinterpret_cast<const u4*>(Ab + kPlaneBytes + off);
        }
    };
    // fp16 scale of the lane's row in slot q, duplicated into both halves
    auto fold_scale = [&](const uint8_t* S, int q) -> uint32_t {
        const uint32_t s16 = *reinterpret_cast<const uint16_t*>(S + soff(q));
        return s16 | (s16 << 16);
    };
    // The chunk's fold scales (slot q), read once per chunk: steps 2q' and 2q' + 1 share a slot
    // when SPC < kSteps.
    uint32_t fsc[MODE == kModeFold ? SPC : 1];
    // fp16 c - 8 of nibble pair s (k-offsets 2s, 2s + 1 of the word's octet): (1024 + c) - 1032,
    // both exact.  The pair mask and the fp16 1024 pair sit in registers the compiler cannot see
    // through, so each pair is one v_and_or_b32 (gfx9 VOP3 operands take no literals: with both
    // as literals every pair cost an AND and an OR).  Not in the 128-row exact-code instances,
    // which are at 256 VGPRs already.
    constexpr bool kRegUnpack = MODE == kModeFold || MI == 2;
    uint32_t nib_mask = 0x000F000Fu, f16_1024 = 0x64006400u;
    if constexpr (kRegUnpack) {
        asm volatile("" : "+s"(nib_mask));
        asm volatile("" : "+v"(f16_1024));
    }
    auto code_pair = [&](uint32_t w, int s) -> h2 {
        const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
        if constexpr (kRegUnpack) return bitcast<h2>(((w >> (4 * s)) & nib_mask) | f16_1024) - off;
        else return codes_minus8_f16(w, s);
    };
    // B fragment of step t from the lane's code word (row n0 + j).
    auto dequant = [&](uint32_t bw, const uint8_t* S, int t, u4& b) {
        if constexpr (MODE == kModeFold) {
            const h2 sc = bitcast<h2>(fsc[(t * SPC) / kSteps]);
            uint32_t p[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) p[s] = bitcast<uint32_t>(code_pair(bw, s) * sc);
            b = u4{p[0], p[1], p[2], p[3]};
        } else if constexpr (XT == kF16) {
            b = u4{bitcast<uint32_t>(code_pair(bw, 0)), bitcast<uint32_t>(code_pair(bw, 1)),
                   bitcast<uint32_t>(code_pair(bw, 2)), bitcast<uint32_t>(code_pair(bw, 3))};
        } else {
            uint32_t X = bw ^ 0x88888888u, Xs = X >> 4;
            asm volatile("" : "+v"(X), "+v"(Xs));   // keeps each conversion one byte select (SDWA)
            b = u4{code_pair_bf16(X, Xs, 0), code_pair_bf16(X, Xs, 1), code_pair_bf16(X, Xs, 2),
                   code_pair_bf16(X, Xs, 3)};
        }
    };
    // Dword e of the B fragment of step t, for interleaving pieces with the MFMAs.  wpre
    // carries per-word values from piece 0 to the later pieces.
    auto dequant_piece = [&](uint32_t w, const uint8_t* S, int t, u4& b, int e, uint32_t (&wpre)[2]) {
        if constexpr (MODE == kModeFold) {
            b[e] = bitcast<uint32_t>(code_pair(w, e) * bitcast<h2>(fsc[(t * SPC) / kSteps]));
        } else if constexpr (XT == kF16) {
            b[e] = bitcast<uint32_t>(code_pair(w, e));
        } else {
            if (e == 0) {
                wpre[0] = w ^ 0x88888888u;
                wpre[1] = wpre[0] >> 4;
                asm volatile("" : "+v"(wpre[0]), "+v"(wpre[1]));   // each conversion stays one byte select (SDWA)
            }
            b[e] = code_pair_bf16(wpre[0], wpre[1], e);
        }
    };
    // One MFMA (two for fp32 x) on tile mi; KIND as below.  An opening step that follows a
    // group (KIND 2) first scales that group's partial sums of tile mi into acc: the rescale of
    // tile mi + 1 then issues while the MFMA of tile mi runs, instead of every wave stalling on
    // its last MFMAs and rescaling all tiles while the matrix unit idles.
    auto mma_tile = [&](const u4& a, const u4& alo, const u4& b, int mi, auto kind) {
        constexpr int K_ = decltype(kind)::value;
        if constexpr (MODE == kModeFold) {
            acc[mi] = mfma32_f16(a, b, acc[mi]);
        } else {
            if constexpr (K_ == 2) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mi][r] = fmaf(part[mi][r], gopen, acc[mi][r]);
                __builtin_amdgcn_sched_barrier(0);   // old partials dead before the MFMA defines new ones
            }
            const f32x16 c0 = (K_ == 0) ? part[mi] : zero16;
            if constexpr (MODE == kModeSplit) part[mi] = mfma32_bf16(alo, b, mfma32_bf16(a, b, c0));
            else if constexpr (XT == kF16) part[mi] = mfma32_f16(a, b, c0);
            else part[mi] = mfma32_bf16(a, b, c0);
        }
    };
    auto flush_open_group = [&]() {
        if constexpr (kGroup) {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mi][r] = fmaf(part[mi][r], gopen, acc[mi][r]);
        }
    };
    // One chunk, software-pipelined: the code words of all steps are read first; while the
    // MFMAs of step t run, the A fragments of step t + 1 are read and its codes unpacked.
    // K0 / K2: kinds of steps 0 and 2 (every other step accumulates; K2 is a group boundary
    // only for gs == 32 in 64-column chunks); fixed at compile time so the chunk body is
    // straight-line code.  Idle waves multiply the valid rows they
    // stream too (their results are never stored): a per-wave branch here would make the
    // accumulators exec-masked.
    auto compute = [&](int st, auto k0, auto k2) {
        constexpr int K0 = decltype(k0)::value, K2 = decltype(k2)::value;
        const uint8_t* Ab = smem + st * kStageBytes + kAOff;
        const uint8_t* Bb = smem + st * kStageBytes + kBOff + wave * kCodeBytes;
        const uint8_t* S = smem + st * kStageBytes + kSOff + (kBlockScales ? 0 : wave * (SPC * 256));
        uint32_t bw[kSteps];
#pragma unroll
        for (int t = 0; t < kSteps; ++t)
            bw[t] = *reinterpret_cast<const uint32_t*>(Bb + 1024 * (t >> 2) + 256 * Rj +
                                                       32 * ((2 * (t & 3) + h + 2 * Rj) & 7) + 4 * (j & 7));
        if constexpr (MODE == kModeFold) {
#pragma unroll
            for (int q = 0; q < SPC; ++q) fsc[q] = fold_scale(S, q);
        }
        u4 a[2][MI], alo[2][MI], b[2];
        read_a(Ab, 0, a[0], alo[0]);
        dequant(bw[0], S, 0, b[0]);
        // Fixed issue order per step: the next step's A reads, then the MFMAs with the next
        // step's unpacking pieces between them (two pieces per MFMA for MI = 2).
        auto one = [&](auto tc, auto kc) {
            constexpr int t = decltype(tc)::value, KIND = decltype(kc)::value;
            if constexpr (t < kSteps - 1) read_a(Ab, t + 1, a[(t + 1) & 1], alo[(t + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            uint32_t wpre[2] = {0u, 0u};
            constexpr int kPer = 4 / MI;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (e % kPer == 0) mma_tile(a[t & 1][e / kPer], alo[t & 1][e / kPer], b[t & 1], e / kPer, kc);
                if constexpr (t < kSteps - 1) dequant_piece(bw[t + 1], S, t + 1, b[(t + 1) & 1], e, wpre);
                if (e % kPer == kPer - 1) __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (KIND != 0) gopen = group_scale(S, (t * SPC) / kSteps);
        };
        typedef std::integral_constant<int, 0> A0;
        one(std::integral_constant<int, 0>{}, k0);
        one(std::integral_constant<int, 1>{}, A0{});
        one(std::integral_constant<int, 2>{}, k2);
        one(std::integral_constant<int, 3>{}, A0{});
        if constexpr (kSteps == 8) {
            one(std::integral_constant<int, 4>{}, A0{});
            one(std::integral_constant<int, 5>{}, A0{});
            one(std::integral_constant<int, 6>{}, A0{});
            one(std::integral_constant<int, 7>{}, A0{});
        }
    };

    // ---------------- pipeline ----------------
    // 16-bit x: chunk c's DMAs (activations, codes, scales) are issued KD chunks ahead; before
    // chunk c is read only the DMAs of the chunks after it may still be in flight.  A chunk
    // staged through the synchronous fallback drained every older load already.
    // fp32 x (KD = 2): codes and scales as above; activations of chunk c + 1 are loaded into
    // registers while chunk c is multiplied and stored after it (the register use retires every
    // older load), so before chunk c is read only those kAUnits loads may be in flight.
    if constexpr (kX16) {
#pragma unroll
        for (int d = 0; d < KD; ++d) {
            if (c_begin + d < c_end) {
                issue_a16(c_begin + d, d);
                issue_codes_scales(c_begin + d, d);
            }
        }
    } else if (c_begin < c_end) {
        issue_codes_scales(c_begin, 0);
        if (c_begin + 1 < c_end) issue_codes_scales(c_begin + 1, 1);
        load_a32(c_begin);
        store_a32(0);
        if (c_begin + 1 < c_end) load_a32(c_begin + 1);
    }
    int st = 0;
    auto chunk = [&](int64_t c, auto k0, auto k2) {
        const int st_next = (st == KD) ? 0 : st + 1;
        const int st_prev = (st == 0) ? KD : st - 1;              // the stage chunk c - 1 used
        if constexpr (kX16) {
            const int64_t ahead = min((int64_t)(KD - 1), c_end - 1 - c);
            if (kBlockScales && wave == 0) wait_chunks_barrier<kDmaPerChunk0, KD - 1>(ahead);
            else wait_chunks_barrier<kDmaPerChunk, KD - 1>(ahead);
            if (c + KD < c_end) {
                issue_a16(c + KD, st_prev);
                issue_codes_scales(c + KD, st_prev);
            }
        } else {
            wait_loads_barrier<kAUnits>();
            if (c + 2 < c_end) issue_codes_scales(c + 2, st_prev);
        }
        compute(st, k0, k2);
        if constexpr (!kX16) {
            if (c + 1 < c_end) {
                store_a32(st_next);
                if (c + 2 < c_end) load_a32(c + 2);
            }
        }
        st = st_next;
    };
    typedef std::integral_constant<int, 0> Acc;        // accumulate into the open group
    typedef std::integral_constant<int, 1> Open;       // open the split's first group
    typedef std::integral_constant<int, 2> Reopen;     // scale the closed group into acc, open the next
    if constexpr (!kGroup) {
        for (int64_t c = c_begin; c < c_end; ++c) chunk(c, Acc{}, Acc{});
    } else if constexpr (SPC == 1) {
        // gs % 64 == 0: a group is cpg whole chunks (the split may start or end inside one);
        // its partial sums are scaled into acc by the first step of the next group, the last
        // group's after the loop
        if (c_begin < c_end) {
            if constexpr (CW == kCKWide) {
                // gs == 128: every chunk opens a group, so the loop is one path (two chunk kinds
                // meeting at the loop head made the compiler copy all partial sums there)
                chunk(c_begin, Open{}, Acc{});
                for (int64_t c = c_begin + 1; c < c_end; ++c) chunk(c, Reopen{}, Acc{});
            } else {
                const int64_t cpg = gs / CW;
                int64_t left = cpg - c_begin % cpg;       // chunks of the open group from c_begin on
                chunk(c_begin, Open{}, Acc{});
                for (int64_t c = c_begin + 1; c < c_end; ++c) {
                    if (--left == 0) {
                        left = cpg;
                        chunk(c, Reopen{}, Acc{});
                    } else {
                        chunk(c, Acc{}, Acc{});
                    }
                }
            }
            flush_open_group();
        }
    } else if (c_begin < c_end) {
        // gs == 32: every 32-column half of a chunk is one group
        chunk(c_begin, Open{}, Reopen{});
        for (int64_t c = c_begin + 1; c < c_end; ++c) chunk(c, Reopen{}, Reopen{});
        flush_open_group();
    }

    // ---------------- epilogue: lane holds D[8 (r/4) + 4 h + r%4][j] of each 32x32 tile ----------------
    // Low-rank term (one split): every wave, idle ones too, stages the block's rows of alpha t, with
    // t[m, j] = sum_s P[(s M + m) rank + j] (chunks in order, zero past M and rank), in the ring's
    // LDS in rows of RP = rank rounded up to 2; the first column tile writes t out.
    const int RP = LR ? (seg.lr.rank + 1) & ~1 : 0;
    const float* Tl = reinterpret_cast<const float*>(smem);
    if constexpr (LR) {
        __syncthreads();                                   // every wave is done with the ring
        float* Tw = reinterpret_cast<float*>(smem);
        const int rank = seg.lr.rank;
        for (int i = tid; i < kBM * RP; i += 64 * kWaves) {
            const int r = i / RP, jj = i - r * RP;
            const int64_t m = m0 + r;
            float v = 0.0f;
            if (m < M && jj < rank) {
                v = chunk_sum<8>(seg.lr.P, seg.lr.chunks, M * rank, m * rank + jj);
                if (seg.lr.Tout && tile == 0) seg.lr.Tout[m * rank + jj] = v;
            }
            Tw[i] = seg.lr.alpha * v;
        }
        __syncthreads();
    }
    if (!wave_active) return;
    if (split_stride) {
        // split partials in the fragment layout: four 16-byte stores per lane and tile, streamed
        // past the caches (the reduction reads each byte once)
        float* plane = seg.out[sg] + (int64_t)z * split_stride;
        const int64_t tn = (seg.col0[sg] + n0) / 32;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int64_t tm = m0 / 32 + mi;
            if (32 * tm >= M) break;
            float* tp = plane + (tm * seg.ntn + tn) * 1024 + 4 * lane;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                __builtin_nontemporal_store(
                    f4{acc[mi][4 * r4], acc[mi][4 * r4 + 1], acc[mi][4 * r4 + 2], acc[mi][4 * r4 + 3]},
                    reinterpret_cast<f4*>(tp + 256 * r4));
        }
        return;
    }
    const int64_t brow = n0 + j;
    float* out = seg.out[sg];
    const int64_t ld = seg.out_ld[sg];
    if constexpr (LR) {
        // acc += (alpha t) G^T on the matrix cores, two ranks per v_mfma_f32_32x32x2_f32: lane l
        // holds A[l % 32][l / 32] (row 32 mi + j of alpha t, rank 2 jp + h) and B[l / 32][l % 32]
        // (G[brow, 2 jp + h]); the result lands in the accumulator layout.  Every lane takes part.
        const int rank = seg.lr.rank;
        const bool col_ok = brow < seg.N[sg];
        for (int jp = 0; jp < RP / 2; ++jp) {
            const int jr = 2 * jp + h;
            const float b = load_sel(seg.lr.G, brow * rank + jr, col_ok && jr < rank);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                acc[mi] = __builtin_amdgcn_mfma_f32_32x32x2f32(Tl[(32 * mi + j) * RP + jr], b, acc[mi], 0, 0, 0);
        }
    }
    if (brow >= seg.N[sg]) return;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + 32 * mi + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m < M) out[m * ld + brow] = acc[mi][r];
        }
    }
}

// ------------------------------------------------------------------------------------------------
bool gemm_fwd_supported(const WView& w, int x_dtype, int fold_ok) {
    if (x_dtype == kF16 && w.scale_f16 && fold_ok) return w.gs % 8 == 0;
    return w.gs % 64 == 0 || w.gs == 32;
}

// Scale slots per chunk of cw columns: one per group that fits a chunk, one per 16 columns for
// fold-mode groups of 8..24 columns (64-column chunks only).
static int fwd_spc(int64_t gs, int cw) {
    if (cw == kCKWide) return gs % 128 == 0 ? 1 : gs % 64 == 0 ? 2 : 4;
    if (gs % 64 == 0) return 1;
    if (gs % 32 == 0) return 2;
    return 4;
}

// K columns per chunk: 128 for the exact-code group mode with gs == 128, where every 128-column
// chunk is one group (measured on a replica of the chunk loop: 1849 against 2383 cycles per 64
// columns, the 64-column loop paying a copy of every partial sum where its two chunk kinds
// meet), and for the fold mode with gs % 32 == 0 (half the waits and barriers per column);
// else 64.
static int fwd_chunk_cols(int mode, int64_t gs) {
    if (mode == kModeGroup && gs == kCKWide) return kCKWide;
    if (mode == kModeFold && gs % 32 == 0) return kCKWide;
    return kCK;
}

// Split count minimising a time model (microseconds): rounds of blocks over the CU slots times
// (chunks per split + fill for pipeline fill and epilogue) at chunk_us per chunk, plus, with splits,
// a reduction launch (~3 us) and the partial buffer written and read back (splits x M x width
// x 8 bytes at ~5 TB/s).  Ties go to fewer splits.  force_splits > 0 takes that count instead
// (clamped to the chunks and rounded to a count without an empty split).
int pick_gemm_splits(int64_t blocks, int64_t n_chunks, int64_t M, int64_t width, int64_t slots, double chunk_us,
                     double* cost_out, int force_splits, double fill) {
    int best = 1;
    double best_cost = 1e300;
    int64_t want = 0;
    if (force_splits > 0) {
        const int64_t f = min((int64_t)force_splits, n_chunks);
        const int64_t per = (n_chunks + f - 1) / f;
        want = (n_chunks + per - 1) / per;
    }
    for (int64_t s = 1; s <= 64 && s <= n_chunks; ++s) {
        const int64_t per = (n_chunks + s - 1) / s;
        if ((n_chunks + per - 1) / per != s) continue;      // some split would be empty
        if (want > 0 && s != want) continue;
        const int64_t rounds = (blocks * s + slots - 1) / slots;
        double cost = chunk_us * (double)rounds * ((double)per + fill);
        if (s > 1) cost += 3.0 + (double)s * (double)M * (double)width * 8.0 / 5e6;
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = (int)s;
        }
    }
    if (cost_out) *cost_out = best_cost;
    return best;
}

// Kernel instance for (activation type, mode, scale slots, scale type, row tiles, fallback, chunk
// columns), handed to f; a combination without an instance hands nothing.
template <int XT, int MODE, int SF, int MI, bool RG, typename F>
static void with_spc(int spc, int cw, bool lr, F&& f) {
    constexpr int KD = XT == kF32 ? 2 : kDepth16;
    if (cw == kCKWide) {
        if constexpr (MODE == kModeGroup) {
            if (spc == 1) {
                if (!lr) f(gemm_fwd_kernel<XT, MODE, 1, SF, MI, KD, RG, kCKWide>);
                else if constexpr (SF == 1) f(gemm_fwd_kernel<XT, MODE, 1, SF, MI, KD, RG, kCKWide, true>);
            }
        } else if constexpr (MODE == kModeFold) {
            if (lr) return;
            if (spc == 1) f(gemm_fwd_kernel<XT, MODE, 1, SF, MI, KD, RG, kCKWide>);
            else if (spc == 2) f(gemm_fwd_kernel<XT, MODE, 2, SF, MI, KD, RG, kCKWide>);
            else f(gemm_fwd_kernel<XT, MODE, 4, SF, MI, KD, RG, kCKWide>);
        }
        return;
    }
    if (lr) return;
    if (spc == 1) f(gemm_fwd_kernel<XT, MODE, 1, SF, MI, KD, RG, kCK>);
    else if (spc == 2) f(gemm_fwd_kernel<XT, MODE, 2, SF, MI, KD, RG, kCK>);
    else if constexpr (MODE == kModeFold) f(gemm_fwd_kernel<XT, MODE, 4, SF, MI, KD, RG, kCK>);
}
template <int XT, int MODE, int SF, typename F>
static void with_mi(int mi, int spc, bool rg, int cw, bool lr, F&& f) {
    if constexpr (MODE == kModeSplit) {
        // 64-row tiles only (see plan_gemm_fwd)
        (void)mi;
        if (rg) with_spc<XT, MODE, SF, 2, true>(spc, cw, lr, f);
        else with_spc<XT, MODE, SF, 2, false>(spc, cw, lr, f);
    } else if (rg) {
        if (mi == 4) with_spc<XT, MODE, SF, 4, true>(spc, cw, lr, f);
        else with_spc<XT, MODE, SF, 2, true>(spc, cw, lr, f);
    } else {
        if (mi == 4) with_spc<XT, MODE, SF, 4, false>(spc, cw, lr, f);
        else with_spc<XT, MODE, SF, 2, false>(spc, cw, lr, f);
    }
}
// lr: the instance with the low-rank epilogue (exact-code group mode, 128-column chunks, fp16
// scales; any other combination hands nothing)
template <typename F>
static void dispatch_fwd(int mode, int x_dtype, int scale_f16, int spc, int mi, bool rg, int cw, F&& f,
                         bool lr = false) {
    if (mode == kModeFold) {
        with_mi<kF16, kModeFold, 1>(mi, spc, rg, cw, lr, f);
    } else if (mode == kModeSplit) {
        if (scale_f16) with_mi<kF32, kModeSplit, 1>(mi, spc, rg, cw, lr, f);
        else with_mi<kF32, kModeSplit, 0>(mi, spc, rg, cw, lr, f);
    } else if (x_dtype == kF16) {
        if (scale_f16) with_mi<kF16, kModeGroup, 1>(mi, spc, rg, cw, lr, f);
        else with_mi<kF16, kModeGroup, 0>(mi, spc, rg, cw, lr, f);
    } else {
        if (scale_f16) with_mi<kBF16, kModeGroup, 1>(mi, spc, rg, cw, lr, f);
        else with_mi<kBF16, kModeGroup, 0>(mi, spc, rg, cw, lr, f);
    }
}

// Blocks of one kernel instance resident per CU (registers and LDS decide), cached per instance.
// Planning may run on several host threads: the cache entries are atomics, and a race only
// repeats the same query.
static int fwd_blocks_per_cu(int mode, int x_dtype, int scale_f16, int spc, int mi, int cw) {
    static std::atomic<int> cache[3][3][2][5][5][2];
    // the aligned instance stands for both fallback variants
    std::atomic<int>& slot = cache[mode][x_dtype][scale_f16 ? 1 : 0][spc][mi][cw == kCKWide ? 1 : 0];
    int n = slot.load(std::memory_order_relaxed);
    if (n == 0) {
        n = 1;
        dispatch_fwd(mode, x_dtype, scale_f16, spc, mi, false, cw, [&](auto kern) {
            int b = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kern, 64 * kWaves, 0) == hipSuccess && b > 0) n = b;
        });
        slot.store(n, std::memory_order_relaxed);
    }
    return n;
}

FwdPlan plan_gemm_fwd(const FwdSeg* segs, int nseg, int x_dtype, int fold_ok, int64_t M, int force_rows,
                      int force_splits) {
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
    const int cw = fwd_chunk_cols(p.mode, w0.gs);
    const int64_t n_chunks = (w0.K + cw - 1) / cw;
    const int spc = fwd_spc(w0.gs, cw);
    double best = 1e300;
    const int forced = force_rows;
    for (int mi : {4, 2}) {
        // fp32 x (hi + lo planes) has no 128-row tile: that instance spilled 250-580 bytes per
        // lane and ran 3-6x slower, so a forced 128 plans 64-row tiles (q4gsw_plan reports it)
        if (mi == 4 && p.mode == kModeSplit) continue;
        if (p.mode != kModeSplit && (forced == 64 || forced == 128) && 32 * mi != forced) continue;
        const int64_t bm = 32 * mi;
        const int64_t blocks = tiles * ((M + bm - 1) / bm);
        const int64_t slots = 256 * (int64_t)fwd_blocks_per_cu(p.mode, x_dtype, w0.scale_f16, spc, mi, cw);
        // a 64-row block does half the MFMA work of a 128-row one per chunk but unpacks as many
        // codes.  Tuned on input sets rotated past the 256 MB Infinity Cache (sweeps on cache-warm
        // inputs favour other split counts).  128-column chunks: fitted to sweeps of row tiles and
        // split counts, 1.75 us per chunk for 128-row tiles (prefill: M = 512, K = 8192, N = 2048,
        // bf16) and 1.3 for 64-row tiles (prefill 1.10-1.21; the fused QKV at M = 128 runs 6 or 8
        // splits 0.3-0.6 us faster than 4), with one chunk of fill; the model then picks the
        // measured best plan for prefill, the fused QKV at M = 128 and 512 and the MLP up
        // projection.
        const bool wide = cw == kCKWide;
        const double chunk_us = wide ? (mi == 4 ? 1.75 : 1.3) : (mi == 4 ? 2.0 : 1.3);
        double cost = 0;
        const int s = pick_gemm_splits(blocks, n_chunks, M, npad_total, slots, chunk_us, &cost, force_splits,
                                       wide ? 1.0 : 2.0);
        if (cost < best - 1e-9) {
            best = cost;
            p.mi = mi;
            p.splits = s;
        }
    }
    p.ws_bytes = p.splits > 1 ? (int64_t)p.splits * frag_plane_floats(M, npad_total) * 4 : 0;
    return p;
}

// One launch over every segment.  With K splits the partials go to ws as splits planes in the
// fragment layout over the columns of all segments (segment i from column sum_{j<i} n_pad_j on).
hipError_t launch_gemm_fwd(const FwdSeg* segs, int nseg, const void* x, int x_dtype, int64_t M,
                           const FwdPlan& plan, float* ws, hipStream_t s, const LowRankEpi* lr, bool* lr_done) {
    if (lr_done) *lr_done = false;
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
            a.out[i] = ws;
            a.col0[i] = col;
        }
        col += segs[i].w.n_pad;
    }
    a.tile_start[nseg] = tiles;
    a.g_pad = w0.g_pad;
    a.ntn = npad_total / 32;
    const int mode = plan.mode;
    const int cw = fwd_chunk_cols(mode, w0.gs);
    const int spc = fwd_spc(w0.gs, cw);
    if (spc == 4 && mode != kModeFold) return hipErrorInvalidValue;
    if ((plan.mi != 4 && plan.mi != 2) || (plan.mi == 4 && mode == kModeSplit)) return hipErrorInvalidValue;
    const int64_t n_chunks = (w0.K + cw - 1) / cw;
    const int per = (int)((n_chunks + plan.splits - 1) / plan.splits);
    const int64_t bm = 32 * plan.mi;
    const int64_t mtiles = (M + bm - 1) / bm;
    const int64_t blocks = tiles * mtiles * plan.splits;
    if (blocks > (int64_t(1) << 24)) return hipErrorInvalidConfiguration;
    const int esize = x_dtype == kF32 ? 4 : 2;
    const int x_fast = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0) && ((w0.K * esize) % 16 == 0);
    const dim3 g((unsigned)blocks);
    const int64_t st = plan.splits == 1 ? 0 : frag_plane_floats(M, npad_total);
    const int64_t K = w0.K, kp = w0.k_pad, gs = w0.gs;
    const int sp = plan.splits, mt = (int)mtiles;
    // XCD-aware order for launches without K splits: the row tile varying fastest put one row
    // tile on each XCD, and every XCD then streamed the whole weight (8.65 MB x 8 of HBM reads
    // at M = 512, K = 2048, N = 8192).  Giving each XCD a contiguous share of the larger operand
    // (the weight, N/2 bytes per k, or the activation, M esize bytes per k) reads it once; the
    // time is the same (the repeats came from the Infinity Cache).  With 2 or 4 splits the same
    // order measured 1% slower (QKV, M = 512), so split launches keep the split index fastest.
    // Only when the pairs divide evenly (the order must stay a bijection).
    a.xcd_g = 1;
    a.xcd_cols = 0;
    if (plan.splits == 1 && (tiles * mtiles) % 8 == 0) {
        a.xcd_g = 8;
        a.xcd_cols = npad_total / 2 >= M * esize;
    }
    if (lr && nseg != 1) return hipErrorInvalidValue;
    const bool rg = !x_fast || (K % cw) != 0;
    // one split: the low-rank term goes into the epilogue where an instance carries it
    bool in_kernel = false;
    if (lr && plan.splits == 1) {
        dispatch_fwd(mode, x_dtype, w0.scale_f16, spc, plan.mi, rg, cw, [&](auto) { in_kernel = true; }, true);
        if (in_kernel) a.lr = *lr;
    }
    bool launched = false;
    dispatch_fwd(mode, x_dtype, w0.scale_f16, spc, plan.mi, rg, cw, [&](auto kern) {
        hipLaunchKernelGGL(kern, g, dim3(64 * kWaves), 0, s, a, x, M, K, kp, gs, x_fast, per, sp, mt, st);
        launched = true;
    }, in_kernel);
    if (!launched) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && in_kernel && lr_done) *lr_done = true;
    if (e != hipSuccess || plan.splits == 1) return e;
    if (lr && lr_done) *lr_done = true;
    const float* ys[3];
    int64_t yld[3], off[3], cols[3];
    int64_t o = 0;
    for (int i = 0; i < nseg; ++i) {
        ys[i] = segs[i].out;
        yld[i] = segs[i].w.N;
        off[i] = o;
        cols[i] = segs[i].w.N;
        o += segs[i].w.n_pad;
    }
    return launch_reduce_frags(ws, plan.splits, M, npad_total, ys, yld, off, cols, nseg, 0, s, lr);
}

}  // namespace q4gsw
