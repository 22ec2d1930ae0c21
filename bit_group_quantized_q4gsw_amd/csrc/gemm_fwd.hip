// MFMA forward for M > 8:  y[m, n] = sum_k x[m, k] * (code[n, k] - 8) * scale[k / gs, n].
//
// The forward GEMM of the pages (the linear_q4gsw op; the WebGPU BK64 QKV PR body
// mirrors the Vulkan q4gsw forward GEMM per projection) re-designed for gfx950:
//
//   * v_mfma_f32_32x32x16 with fp32 accumulators; a wave owns a 128 (M) x 64 (N) output
//     tile = 4 x 2 MFMA tiles, so every dequantised code feeds 128 activation rows;
//   * block = 4 waves side by side in N (block tile 128 x 256), one block per CU;
//   * every global read is an LDS-DMA (global_load_lds): the 64-column activation chunk
//     (shared by the 4 waves), each wave's 2 KB of codes and its scales travel straight
//     into a ring of kStages LDS stages, kDepth chunks ahead of the MFMAs, with no VGPR
//     staging.  Explicit vmcnt waits + s_barrier order the ring; the compiler only sees
//     LDS reads (fp32 activations are the exception: split into bf16 hi + lo planes in
//     registers on their way into LDS);
//   * LDS swizzles: activation k-octet slots of row r sit at slot (octet ^ ((r >> 1) & 7)),
//     so the 16 lanes of an A-fragment read phase (16 rows of 128 bytes) cover all 64
//     banks; the 256-byte code run of row-octet R is rotated by R 32-byte blocks, so the 32
//     lanes reading one k-octet of 8 row-octets hit 8 distinct bank groups;
//   * the K range is split across blocks when the output tiles cannot fill the GPU; the
//     split index is the fastest-varying block coordinate, so with 8 splits every XCD owns
//     one K slice (its activation and code slices stay in that XCD's L2); a reduction
//     kernel sums the split partials.
//
// K order inside a 64-column chunk: MFMA step t contracts k-octets 2t (lanes 0..31) and
// 2t+1 (lanes 32..63), so a step covers 16 consecutive columns.
//
// Precision routes (all with fp32 accumulation):
//   kModeFold  (fp16 x, fp16 scales checked foldable at pack time):
//       B = fp16((code - 8) * scale), one rounding, |err| <= 2^-11 |w|.
//   kModeGroup (fp16 or bf16 x): B = code - 8 held exactly (fp16, or bf16 of 16 (code - 8))
//       and the scale multiplies the fp32 partial sum of each scale group, which the MFMAs
//       build in a separate set of accumulators.
//   kModeSplit (fp32 x): x = hi + lo in bf16 (|err| <= 2^-18 |x|), two MFMA passes
//       against the exact bf16 codes, scale per group as in kModeGroup.
#include "device.h"
#include "internal.h"

#include <type_traits>

namespace q4gsw {

constexpr int kBM = 128;            // block rows (M)
constexpr int kWN = 64;             // wave columns (N)
constexpr int kBN = 4 * kWN;        // block columns (N)
constexpr int kCK = 64;             // K columns per chunk
constexpr int kDepth = 2;           // chunks in flight ahead of the chunk being multiplied
constexpr int kStages = kDepth + 1; // LDS stages in the ring
constexpr int kRowBytes = 128;      // one 16-bit activation row of a chunk in LDS
constexpr int kPlaneBytes = kBM * kRowBytes;
constexpr int kCodeBytes = 2048;    // one wave's codes for one chunk: 64 rows x 64 columns x 4 bits

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

// bf16 pair (16 (c_lo - 8), 16 (c_hi - 8)) for the four MFMA dwords of a code word.  H holds
// 16 x the odd nibble positions and L 16 x the even ones as signed bytes; byte b of H is
// position 2b + 1, byte b of L position 2b.  Dword e needs positions e and e + 4.
__device__ __forceinline__ u4 codes16_bf16(uint32_t w) {
    const uint32_t wx = w ^ 0x88888888u;
    uint32_t H = wx & 0xF0F0F0F0u;
    uint32_t L = (wx << 4) & 0xF0F0F0F0u;
    // opaque to the optimiser, so each value below stays one byte-select (SDWA) conversion
    asm volatile("" : "+v"(H), "+v"(L));
    const float p0 = (float)(int8_t)(L & 0xFFu), p4 = (float)(int8_t)((L >> 16) & 0xFFu);
    const float p1 = (float)(int8_t)(H & 0xFFu), p5 = (float)(int8_t)((H >> 16) & 0xFFu);
    const float p2 = (float)(int8_t)((L >> 8) & 0xFFu), p6 = (float)(int8_t)(L >> 24);
    const float p3 = (float)(int8_t)((H >> 8) & 0xFFu), p7 = (float)(int8_t)(H >> 24);
    const uint32_t sel = 0x07060302u;     // upper halves: small integers are exact in bf16
    return u4{__builtin_amdgcn_perm(bitcast<uint32_t>(p4), bitcast<uint32_t>(p0), sel),
              __builtin_amdgcn_perm(bitcast<uint32_t>(p5), bitcast<uint32_t>(p1), sel),
              __builtin_amdgcn_perm(bitcast<uint32_t>(p6), bitcast<uint32_t>(p2), sel),
              __builtin_amdgcn_perm(bitcast<uint32_t>(p7), bitcast<uint32_t>(p3), sel)};
}

__device__ __forceinline__ u4 codes_f16(uint32_t w) {
    return u4{bitcast<uint32_t>(codes_minus8_f16(w, 0)), bitcast<uint32_t>(codes_minus8_f16(w, 1)),
              bitcast<uint32_t>(codes_minus8_f16(w, 2)), bitcast<uint32_t>(codes_minus8_f16(w, 3))};
}

// SPC: scale slots per chunk (1: gs % 64 == 0; 2: gs % 32 == 0, one slot per 32 columns, which
// the group and split modes take only for gs == 32; 4: fold mode with any gs % 8 == 0, one slot
// per k-octet of the lane).  SF: 1 = fp16 scales.
template <int XT, int MODE, int SPC, int SF>
__global__ __launch_bounds__(256, 1) void gemm_fwd_kernel(FwdSegArgs seg, const void* __restrict__ x, int64_t M,
                                                          int64_t K, int64_t k_pad, int64_t gs, int x_fast,
                                                          int chunks_per_split, int splits, int mtiles,
                                                          int64_t split_stride) {
    constexpr bool kX16 = XT != kF32;
    constexpr int kPlanes = kX16 ? 1 : 2;
    constexpr int kADma = kX16 ? 4 : 0;                   // activation DMAs per wave per chunk
    constexpr int kSDma = SF ? SPC : 2 * SPC;             // scale DMAs per wave per chunk
    constexpr int kDmaPerChunk = kADma + 2 + kSDma;
    constexpr int kAOff = 0;
    constexpr int kBOff = kPlanes * kPlaneBytes;
    constexpr int kSOff = kBOff + 4 * kCodeBytes;
    constexpr int kStageBytes = kSOff + 4 * kSDma * 256;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 31;          // MFMA row / column inside a 32x32 tile
    const int h = lane >> 5;          // MFMA k-group: k-octet 2t + h of step t

    // ---- block -> (K split, M tile, N tile); the split index varies fastest ----
    const int64_t bid = blockIdx.x;
    const int z = (int)(bid % splits);
    const int64_t rest = bid / splits;
    const int64_t mb = rest % mtiles;
    const int64_t tile = rest / mtiles;
    int sg = 0;
    while (sg + 1 < seg.nseg && tile >= seg.tile_start[sg + 1]) ++sg;
    const int64_t n0 = (tile - seg.tile_start[sg]) * kBN + (int64_t)wave * kWN;   // first W row of the wave
    const bool wave_active = n0 < seg.n_pad[sg];
    const int64_t nw = wave_active ? n0 : 0;   // an idle wave streams valid rows it never uses
    const int64_t m0 = mb * kBM;
    const int64_t kocts = k_pad >> 3;
    const int64_t n_chunks = (K + kCK - 1) / kCK;
    const int64_t c_begin = (int64_t)z * chunks_per_split;
    const int64_t c_end = min(c_begin + (int64_t)chunks_per_split, n_chunks);

    lds_u8* const sm_l = (lds_u8*)smem;

    // ---------------- DMA source addresses ----------------
    // Codes: DMA r of a wave covers row-octets 4r .. 4r+3 of the wave; lane l fills LDS
    // bytes 16 l of it = row-octet R = 4r + (l >> 4), rotated block slot p = (l & 15) >> 1,
    // half l & 1, which holds k-octet (p - R) & 7 of the chunk.
    const uint8_t* csrc[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int R = 4 * r + (lane >> 4);
        const int p = (lane & 15) >> 1;
        const int o = (p - R) & 7;
        csrc[r] = seg.nib[sg] + 32 * (((nw >> 3) + R) * kocts + o) + 16 * (lane & 1);
    }
    // Scales: lane (j, h) loads the scales of W rows nw + 2j, nw + 2j + 1 (adjacent in the
    // scale plane) for each of its slots.
    const int64_t srow = nw + 2 * j;
    const int64_t sbase = (srow >> 3) * (seg.g_pad * 8) + (srow & 7);
    const uint8_t* sptr = static_cast<const uint8_t*>(seg.scales[sg]);
    // Activations (16-bit): DMA q of wave w covers rows 32w + 8q .. +7; lane i fills slot i & 7
    // of row (i >> 3), which holds k-octet (i & 7) ^ ((row >> 1) & 7).
    const uint16_t* xa[4];
    int xoct[4];
    if constexpr (kX16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = 32 * wave + 8 * q + (lane >> 3);
            xoct[q] = (lane & 7) ^ ((row >> 1) & 7);
            const int64_t m = min(m0 + row, M - 1);     // rows past M only feed discarded outputs
            xa[q] = static_cast<const uint16_t*>(x) + m * K + 8 * xoct[q];
        }
    }

    auto issue_codes_scales = [&](int64_t c, int st) {
        lds_u8* base = sm_l + st * kStageBytes;
#pragma unroll
        for (int r = 0; r < 2; ++r) dma16(csrc[r] + 256 * c, base + kBOff + wave * kCodeBytes + 1024 * r);
        const uint32_t kc = (uint32_t)(c * kCK);
        const uint32_t ug = (uint32_t)gs;
#pragma unroll
        for (int q = 0; q < SPC; ++q) {
            const uint32_t k = (SPC == 4) ? kc + 16 * q + 8 * h : kc + 32 * q;
            const int64_t idx = sbase + (int64_t)(k / ug) * 8;
            lds_u8* sdst = base + kSOff + wave * (kSDma * 256);
            if constexpr (SF) {
                dma4(sptr + 2 * idx, sdst + 256 * q);
            } else {
                dma4(sptr + 4 * idx, sdst + 256 * (2 * q));
                dma4(sptr + 4 * idx + 4, sdst + 256 * (2 * q + 1));
            }
        }
    };
    // Synchronous fallback for a ragged K tail or unaligned x: zero-filled register loads
    // into the slots the DMA would write.
    auto fill_a16_slow = [&](int64_t kc, int st) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = 32 * wave + 8 * q + (lane >> 3);
            const int64_t m = m0 + row;
            const int64_t k = kc + 8 * xoct[q];
            uint32_t e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                e[i] = (m < M && k + i < K) ? static_cast<const uint16_t*>(x)[m * K + k + i] : 0u;
            *reinterpret_cast<u4*>(smem + st * kStageBytes + kAOff + row * kRowBytes + 16 * (lane & 7)) =
                u4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
        }
    };
    auto issue_a16 = [&](int64_t c, int st) {
        const int64_t kc = c * kCK;
        if (x_fast && kc + kCK <= K) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dma16(xa[q] + kc, sm_l + st * kStageBytes + kAOff + (32 * wave + 8 * q) * kRowBytes);
        } else {
            fill_a16_slow(kc, st);
        }
    };

    // fp32 activations: 8 float4 units per thread, split into bf16 hi / lo planes at store time.
    f4 areg[8];
    auto load_a32 = [&](int64_t c) {
        const int64_t kc = c * kCK;
        const bool fast = x_fast && kc + kCK <= K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int unit = tid + 256 * i;
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
        for (int i = 0; i < 8; ++i) {
            const int unit = tid + 256 * i;
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
    f32x16 acc[4][2];
    f32x16 part[kGroup ? 4 : 1][2];          // partial sums of the open scale group
    float gopen[2] = {0.f, 0.f};             // its scales (rows brow, brow + 1)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][u][r] = 0.f;
    const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // ---------------- one chunk of MFMAs ----------------
    const int swz = (j >> 1) & 7;     // ((row >> 1) & 7) of every A row this lane reads
    const int Rl = j >> 2;            // this lane's row-octet inside the wave
    // fp32 group scale of slot q for rows brow (u = 0) and brow + 1 (u = 1); bf16 codes carry
    // a factor 16 that the scale removes exactly.
    auto group_scale = [&](const uint8_t* S, int q, float (&g)[2]) {
        constexpr float kUnit = (XT == kF16) ? 1.0f : 0.0625f;
        if constexpr (SF) {
            const uint32_t sv = *reinterpret_cast<const uint32_t*>(S + 256 * q + 4 * lane);
            g[0] = (float)bitcast<_Float16>((uint16_t)(sv & 0xFFFFu)) * kUnit;
            g[1] = (float)bitcast<_Float16>((uint16_t)(sv >> 16)) * kUnit;
        } else {
            g[0] = *reinterpret_cast<const float*>(S + 256 * (2 * q) + 4 * lane) * kUnit;
            g[1] = *reinterpret_cast<const float*>(S + 256 * (2 * q + 1) + 4 * lane) * kUnit;
        }
    };
    // A fragments of step t for the wave's four 32-row tiles (and the lo plane for fp32 x).
    auto read_a = [&](const uint8_t* Ab, int t, u4 (&a)[4], u4 (&alo)[4]) {
        const int slot = 16 * ((2 * t + h) ^ swz);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int off = (32 * mi + j) * kRowBytes + slot;
            a[mi] = *reinterpret_cast<const u4*>(Ab + off);
            if constexpr (MODE == kModeSplit) alo[mi] = *reinterpret_cast<const u4*>(Ab + kPlaneBytes + off);
        }
    };
    // B fragments of step t from the lane's code words (rows brow, brow + 1).
    auto dequant = [&](u2 bw, const uint8_t* S, int t, u4 (&b)[2]) {
        if constexpr (MODE == kModeFold) {
            const uint32_t sv = *reinterpret_cast<const uint32_t*>(S + 256 * ((t * SPC) / 4) + 4 * lane);
            const h2 s0 = bitcast<h2>((sv & 0xFFFFu) | (sv << 16));
            const h2 s1 = bitcast<h2>((sv >> 16) | (sv & 0xFFFF0000u));
            uint32_t p0[4], p1[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                p0[s] = bitcast<uint32_t>(codes_minus8_f16(bw.x, s) * s0);
                p1[s] = bitcast<uint32_t>(codes_minus8_f16(bw.y, s) * s1);
            }
            b[0] = u4{p0[0], p0[1], p0[2], p0[3]};
            b[1] = u4{p1[0], p1[1], p1[2], p1[3]};
        } else if constexpr (XT == kF16) {
            b[0] = codes_f16(bw.x);
            b[1] = codes_f16(bw.y);
        } else {
            b[0] = codes16_bf16(bw.x);
            b[1] = codes16_bf16(bw.y);
        }
    };
    // Dword e of B fragment u of step t (piece i = 4 u + e of the step's unpacking), for
    // interleaving one piece after each MFMA.  wpre[u] carries per-word values from piece
    // 4 u to the later pieces of the same word.
    auto dequant_piece = [&](u2 bw, const uint8_t* S, int t, u4 (&b)[2], int i, uint32_t (&wpre)[2][2]) {
        const int u = i >> 2, e = i & 3;
        const uint32_t w = u ? bw.y : bw.x;
        if constexpr (MODE == kModeFold) {
            if (e == 0) wpre[u][0] = *reinterpret_cast<const uint32_t*>(S + 256 * ((t * SPC) / 4) + 4 * lane);
            const uint32_t sv = wpre[u][0];
            const h2 sc = u ? bitcast<h2>((sv >> 16) | (sv & 0xFFFF0000u)) : bitcast<h2>((sv & 0xFFFFu) | (sv << 16));
            b[u][e] = bitcast<uint32_t>(codes_minus8_f16(w, e) * sc);
        } else if constexpr (XT == kF16) {
            b[u][e] = bitcast<uint32_t>(codes_minus8_f16(w, e));
        } else {
            if (e == 0) {
                const uint32_t wx = w ^ 0x88888888u;
                wpre[u][0] = wx & 0xF0F0F0F0u;
                wpre[u][1] = (wx << 4) & 0xF0F0F0F0u;
                asm volatile("" : "+v"(wpre[u][0]), "+v"(wpre[u][1]));
            }
            // dword e holds nibble positions e (low half) and e + 4 (high half); even positions
            // come from L = wpre[1], odd ones from H = wpre[0], byte (position >> 1)
            const uint32_t src = (e & 1) ? wpre[u][0] : wpre[u][1];
            const int by = e >> 1;
            const float lo = (float)(int8_t)((src >> (8 * by)) & 0xFFu);
            const float hi = (float)(int8_t)((src >> (8 * (by + 2))) & 0xFFu);
            b[u][e] = __builtin_amdgcn_perm(bitcast<uint32_t>(hi), bitcast<uint32_t>(lo), 0x07060302u);
        }
    };
    // One MFMA (two for fp32 x) on tile (mi, u); KIND as below.
    auto mma_tile = [&](const u4& a, const u4& alo, const u4& bu, int mi, int u, auto kind) {
        constexpr int K_ = decltype(kind)::value;
        if constexpr (MODE == kModeFold) {
            acc[mi][u] = mfma32_f16(a, bu, acc[mi][u]);
        } else {
            const f32x16 c0 = (K_ == 0) ? part[mi][u] : zero16;
            if constexpr (MODE == kModeSplit) part[mi][u] = mfma32_bf16(alo, bu, mfma32_bf16(a, bu, c0));
            else if constexpr (XT == kF16) part[mi][u] = mfma32_f16(a, bu, c0);
            else part[mi][u] = mfma32_bf16(a, bu, c0);
        }
    };
    auto flush_open_group = [&]() {
        if constexpr (kGroup) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mi][u][r] = fmaf(part[mi][u][r], gopen[u], acc[mi][u][r]);
        }
    };
    // One chunk, software-pipelined: the code words of all four steps are read first; while
    // the MFMAs of step t run, the A fragments of step t + 1 are read and its codes unpacked.
    // K0 / K2: kinds of steps 0 and 2 (steps 1 and 3 always accumulate); fixed at compile
    // time so the chunk body is straight-line code.  Idle waves multiply the valid rows they
    // stream too (their results are never stored): a per-wave branch here would make the
    // accumulators exec-masked.
    auto compute = [&](int st, auto k0, auto k2) {
        constexpr int K0 = decltype(k0)::value, K2 = decltype(k2)::value;
        const uint8_t* Ab = smem + st * kStageBytes + kAOff;
        const uint8_t* Bb = smem + st * kStageBytes + kBOff + wave * kCodeBytes;
        const uint8_t* S = smem + st * kStageBytes + kSOff + wave * (kSDma * 256);
        u2 bw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            bw[t] = *reinterpret_cast<const u2*>(Bb + 256 * Rl + 32 * ((2 * t + h + Rl) & 7) + 8 * (j & 3));
        u4 a[2][4], alo[2][4], b[2][2];
        read_a(Ab, 0, a[0], alo[0]);
        dequant(bw[0], S, 0, b[0]);
        // Fixed issue order per step: the next step's A reads, then eight (MFMA, unpacking
        // piece) pairs, so the single wave keeps the VALU busy while the matrix core runs and
        // the A reads have a whole step to land.
        auto one = [&](auto tc, auto kc) {
            constexpr int t = decltype(tc)::value, KIND = decltype(kc)::value;
            if constexpr (t < 3) read_a(Ab, t + 1, a[(t + 1) & 1], alo[(t + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            uint32_t wpre[2][2] = {{0u, 0u}, {0u, 0u}};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                mma_tile(a[t & 1][i >> 1], alo[t & 1][i >> 1], b[t & 1][i & 1], i >> 1, i & 1, kc);
                if constexpr (t < 3) dequant_piece(bw[t + 1], S, t + 1, b[(t + 1) & 1], (i & 1) * 4 + (i >> 1), wpre);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (KIND != 0) group_scale(S, SPC == 2 ? (t >> 1) : 0, gopen);
            if constexpr (kGroup && SPC == 2 && (t & 1)) flush_open_group();   // gs == 32
        };
        one(std::integral_constant<int, 0>{}, k0);
        one(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
        one(std::integral_constant<int, 2>{}, k2);
        one(std::integral_constant<int, 3>{}, std::integral_constant<int, 0>{});
    };

    // ---------------- pipeline ----------------
    // 16-bit x: chunk c's DMAs (activations, codes, scales) are issued kDepth chunks ahead;
    // before chunk c is read only chunk c + 1's DMAs may still be in flight.  A chunk staged
    // through the synchronous fallback drained every older load already.
    // fp32 x: codes and scales as above; activations of chunk c + 1 are loaded into registers
    // while chunk c is multiplied and stored after it (the register use retires every older
    // load), so before chunk c is read only those 8 loads may be in flight.
    static_assert(kDepth == 2, "wait counts and stage rotation assume two chunks in flight");
    if (c_begin < c_end) {
        if constexpr (kX16) issue_a16(c_begin, 0);
        issue_codes_scales(c_begin, 0);
        if (c_begin + 1 < c_end) {
            if constexpr (kX16) issue_a16(c_begin + 1, 1);
            issue_codes_scales(c_begin + 1, 1);
        }
        if constexpr (!kX16) {
            load_a32(c_begin);
            store_a32(0);
            if (c_begin + 1 < c_end) load_a32(c_begin + 1);
        }
    }
    int st = 0;
    auto chunk = [&](int64_t c, auto k0, auto k2) {
        const int st_next = (st == 2) ? 0 : st + 1;
        const int st_prev = (st == 0) ? 2 : st - 1;
        if constexpr (kX16) {
            if (c + 1 < c_end) wait_loads_barrier<kDmaPerChunk>();
            else wait_loads_barrier<0>();
            if (c + kDepth < c_end) {
                issue_a16(c + kDepth, st_prev);                   // the stage chunk c - 1 used
                issue_codes_scales(c + kDepth, st_prev);
            }
        } else {
            wait_loads_barrier<8>();
            if (c + kDepth < c_end) issue_codes_scales(c + kDepth, st_prev);
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
    typedef std::integral_constant<int, 0> Acc;      // accumulate into the open group
    typedef std::integral_constant<int, 1> Open;     // open the split's first group
    if constexpr (!kGroup) {
        for (int64_t c = c_begin; c < c_end; ++c) chunk(c, Acc{}, Acc{});
    } else if constexpr (SPC == 1) {
        // gs % 64 == 0: a group is cpg whole chunks (the split may start or end inside one);
        // its partial sums are scaled into acc after its last chunk
        const int64_t cpg = gs / kCK;
        int64_t c = c_begin;
        while (c < c_end) {
            const int64_t gend = min(c_end, (c / cpg + 1) * cpg);
            chunk(c, Open{}, Acc{});
            for (++c; c < gend; ++c) chunk(c, Acc{}, Acc{});
            flush_open_group();
        }
    } else {
        // gs == 32: every 32-column half of a chunk is one group, scaled in inside the chunk
        for (int64_t c = c_begin; c < c_end; ++c) chunk(c, Open{}, Open{});
    }

    // ---------------- epilogue: lane holds D[8 (r/4) + 4 h + r%4][j] of each 32x32 tile ----------------
    if (!wave_active) return;
    const int64_t brow = n0 + 2 * j;
    float* out = seg.out[sg] + (int64_t)z * split_stride;
    const int64_t ld = seg.out_ld[sg];
    const int64_t ncols = split_stride ? seg.n_pad[sg] : seg.N[sg];
    const bool pair_ok = (ld % 2 == 0) && (brow + 2 <= ncols);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + 32 * mi + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m >= M) continue;
            float* dst = out + m * ld + brow;
            if (pair_ok) {
                *reinterpret_cast<float2*>(dst) = make_float2(acc[mi][0][r], acc[mi][1][r]);
            } else {
                if (brow < ncols) dst[0] = acc[mi][0][r];
                if (brow + 1 < ncols) dst[1] = acc[mi][1][r];
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
bool gemm_fwd_supported(const WView& w, int x_dtype, int fold_ok) {
    if (x_dtype == kF16 && w.scale_f16 && fold_ok) return w.gs % 8 == 0;
    return w.gs % 64 == 0 || w.gs == 32;
}

static int fwd_spc(int64_t gs) {
    if (gs % 64 == 0) return 1;
    if (gs % 32 == 0) return 2;
    return 4;
}

// Split count minimising a time model (microseconds): rounds of blocks over the 256 CUs times
// (chunks per split + 2 for pipeline fill and epilogue) at ~2 us per chunk, plus, with splits,
// a reduction launch (~3 us) and the partial buffer written and read back (splits x M x width
// x 8 bytes at ~5 TB/s).  Ties go to fewer splits.
int pick_gemm_splits(int64_t blocks, int64_t n_chunks, int64_t M, int64_t width) {
    const int64_t cus = 256;
    int best = 1;
    double best_cost = 1e300;
    for (int64_t s = 1; s <= 64 && s <= n_chunks; ++s) {
        const int64_t per = (n_chunks + s - 1) / s;
        if ((n_chunks + per - 1) / per != s) continue;      // some split would be empty
        const int64_t rounds = (blocks * s + cus - 1) / cus;
        double cost = 2.0 * (double)rounds * (double)(per + 2);
        if (s > 1) cost += 3.0 + (double)s * (double)M * (double)width * 8.0 / 5e6;
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = (int)s;
        }
    }
    return best;
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
    const int64_t n_chunks = (w0.K + kCK - 1) / kCK;
    const int splits = pick_gemm_splits(blocks, n_chunks, M, npad_total);
    p.splits = splits;
    p.ws_bytes = splits > 1 ? (int64_t)splits * M * npad_total * 4 : 0;
    return p;
}

template <int XT, int MODE, int SPC, int SF>
static void launch_fwd_t(dim3 grid, hipStream_t s, const FwdSegArgs& a, const void* x, int64_t M, int64_t K,
                         int64_t k_pad, int64_t gs, int x_fast, int per, int splits, int mtiles,
                         int64_t stride) {
    hipLaunchKernelGGL((gemm_fwd_kernel<XT, MODE, SPC, SF>), grid, dim3(256), 0, s, a, x, M, K, k_pad, gs, x_fast,
                       per, splits, mtiles, stride);
}

template <int XT, int MODE, int SF>
static void launch_fwd_spc(int spc, dim3 grid, hipStream_t s, const FwdSegArgs& a, const void* x, int64_t M,
                           int64_t K, int64_t k_pad, int64_t gs, int x_fast, int per, int splits, int mtiles,
                           int64_t stride) {
    if (spc == 1) launch_fwd_t<XT, MODE, 1, SF>(grid, s, a, x, M, K, k_pad, gs, x_fast, per, splits, mtiles, stride);
    else if (spc == 2) launch_fwd_t<XT, MODE, 2, SF>(grid, s, a, x, M, K, k_pad, gs, x_fast, per, splits, mtiles, stride);
    else if constexpr (MODE == kModeFold)
        launch_fwd_t<XT, MODE, 4, SF>(grid, s, a, x, M, K, k_pad, gs, x_fast, per, splits, mtiles, stride);
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
    const int spc = fwd_spc(w0.gs);
    if (spc == 4 && mode != kModeFold) return hipErrorInvalidValue;
    const int64_t n_chunks = (w0.K + kCK - 1) / kCK;
    const int per = (int)((n_chunks + plan.splits - 1) / plan.splits);
    const int64_t mtiles = (M + kBM - 1) / kBM;
    const int64_t blocks = tiles * mtiles * plan.splits;
    if (blocks > (int64_t(1) << 24)) return hipErrorInvalidConfiguration;
    const int esize = x_dtype == kF32 ? 4 : 2;
    const int x_fast = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0) && ((w0.K * esize) % 16 == 0);
    const dim3 g((unsigned)blocks);
    const int64_t st = plan.splits == 1 ? 0 : M * npad_total;
    const int64_t K = w0.K, kp = w0.k_pad, gs = w0.gs;
    const int sp = plan.splits, mt = (int)mtiles;
    if (mode == kModeFold) {
        launch_fwd_spc<kF16, kModeFold, 1>(spc, g, s, a, x, M, K, kp, gs, x_fast, per, sp, mt, st);
    } else if (mode == kModeSplit) {
        if (w0.scale_f16) launch_fwd_spc<kF32, kModeSplit, 1>(spc, g, s, a, x, M, K, kp, gs, x_fast, per, sp, mt, st);
        else launch_fwd_spc<kF32, kModeSplit, 0>(spc, g, s, a, x, M, K, kp, gs, x_fast, per, sp, mt, st);
    } else if (x_dtype == kF16) {
        if (w0.scale_f16) launch_fwd_spc<kF16, kModeGroup, 1>(spc, g, s, a, x, M, K, kp, gs, x_fast, per, sp, mt, st);
        else launch_fwd_spc<kF16, kModeGroup, 0>(spc, g, s, a, x, M, K, kp, gs, x_fast, per, sp, mt, st);
    } else {
        if (w0.scale_f16) launch_fwd_spc<kBF16, kModeGroup, 1>(spc, g, s, a, x, M, K, kp, gs, x_fast, per, sp, mt, st);
        else launch_fwd_spc<kBF16, kModeGroup, 0>(spc, g, s, a, x, M, K, kp, gs, x_fast, per, sp, mt, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
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
    return launch_reduce_segments(ws, plan.splits, M, npad_total, ys, yld, off, cols, nseg, s);
}

}  // namespace q4gsw
