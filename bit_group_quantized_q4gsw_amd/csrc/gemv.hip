// Small-M (decode, M <= 8) q4gsw kernels: bandwidth-bound streaming over the packed codes.
//
// Forward:   y[m, n]   = sum_k x[m, k] * (code[n, k] - 8) * scale[k / gs, n]
// Backward:  d_x[m, k] = sum_n d_out[m, n] * (code[n, k] - 8) * scale[k / gs, n]
// (the input gradient of the Vulkan q4gsw-backward PR body, contracting over N).
//
// Every lane reads whole 32-byte micro-blocks (8 rows x 8 columns of codes) with two
// 16-byte loads; a wave's 64 lanes cover 4 row-octets x 16 k-octets, i.e. four
// contiguous 512-byte runs.  Codes are unpacked in registers to the exact values
// c - 8, products are fp32 (or fp16 pairs with fp32 dot2 accumulation for fp16
// activations), and partial sums are reduced across lanes with register-to-register
// cross-lane operations (DPP and the gfx950 row and half swaps) and across waves in LDS.
// A code 8 therefore contributes exactly 0.
// Requires group_size % 8 == 0 so a k-octet lies inside one scale group.
#include "device.h"
#include "internal.h"

#include <type_traits>

namespace q4gsw {

namespace {

__device__ __forceinline__ void load_micro_block(const uint8_t* p, uint32_t (&wd)[8]) {
    const u4 a = ldg16_stream(p);
    const u4 b = ldg16_stream(p + 16);
    wd[0] = a.x; wd[1] = a.y; wd[2] = a.z; wd[3] = a.w;
    wd[4] = b.x; wd[5] = b.y; wd[6] = b.z; wd[7] = b.w;
}

// Eight consecutive scales scale[g, n0 .. n0+7] as fp32.
__device__ __forceinline__ void load_scales8(const void* plane, int scale_f16, int64_t idx, float (&sc)[8]) {
    if (scale_f16) {
        const u4 v = ldg16(static_cast<const uint16_t*>(plane) + idx);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[2 * i] = f16_bits_to_f32((uint16_t)(u[i] & 0xFFFFu));
            sc[2 * i + 1] = f16_bits_to_f32((uint16_t)(u[i] >> 16));
        }
    } else {
        const f4 a = *reinterpret_cast<const f4*>(static_cast<const float*>(plane) + idx);
        const f4 b = *reinterpret_cast<const f4*>(static_cast<const float*>(plane) + idx + 4);
        sc[0] = a.x; sc[1] = a.y; sc[2] = a.z; sc[3] = a.w;
        sc[4] = b.x; sc[5] = b.y; sc[6] = b.z; sc[7] = b.w;
    }
}

// Eight activation values src[base + 0..7] widened to fp32; elements at or past `limit` read as 0.
template <int DT>
__device__ __forceinline__ void load_act8(const void* src, int64_t base, int64_t pos, int64_t limit, int vec,
                                          float (&v)[8]) {
    if (vec && pos + 8 <= limit) {
        if constexpr (DT == kF32) {
            const f4 a = *reinterpret_cast<const f4*>(static_cast<const float*>(src) + base);
            const f4 b = *reinterpret_cast<const f4*>(static_cast<const float*>(src) + base + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
            const u4 a = ldg16(static_cast<const uint16_t*>(src) + base);
            const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (DT == kF16) {
                    v[2 * i] = f16_bits_to_f32((uint16_t)(u[i] & 0xFFFFu));
                    v[2 * i + 1] = f16_bits_to_f32((uint16_t)(u[i] >> 16));
                } else {
                    v[2 * i] = bitcast<float>(u[i] << 16);
                    v[2 * i + 1] = bitcast<float>(u[i] & 0xFFFF0000u);
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (pos + j < limit) ? load_elem<DT>(src, base + j) : 0.0f;
    }
}

}  // namespace

// Grid: (n_pad / 8, splits).  Block: W waves (64 * W threads; W <= 16 for M <= 4, else 8).  A
// block owns one row-octet (8 rows).  Each load instruction of a wave reads 1 KB of contiguous codes: lane l
// takes bytes [16 l, 16 l + 16) of a 32-micro-block run, i.e. rows 4 (l & 1) .. +3 of
// k-octet l / 2.  A wave takes 64 k-octets per iteration (two loads per lane, both issued
// before any unpacking) and the W waves of a block take adjacent 512-column slices, so a
// decode launch is many small blocks that each stream one contiguous row-octet.
//
// One launch serves up to three weights sharing K, group size and scale dtype (the small-M fused
// QKV): blocks [blk_start[i], blk_start[i + 1]) take the row-octets of weight i and do exactly
// the work of a launch for that weight alone.
struct GemvSegs {
    WView w[3];
    float* out[3];
    int64_t out_ld[3];           // row pitch of each output
    int64_t row_limit[3];        // rows stored (N unsplit, n_pad into a split workspace)
    int64_t blk_start[4];        // first block of each weight; blk_start[nseg] = grid.x
    int nseg;
};

// Most waves per block for MT activation rows: up to four rows fit 128 VGPRs (16 waves, 1024
// threads); more rows take a 512-thread bound (256 VGPRs), which a 1024-thread one made spill.
constexpr int gemv_fwd_max_waves(int64_t mt) { return mt <= 4 ? 16 : 8; }

template <int MT, int XT, int SF>
__global__ __launch_bounds__(64 * gemv_fwd_max_waves(MT)) void gemv_fwd_kernel(GemvSegs segs, const void* __restrict__ x, int x_vec,
                                                        int64_t split_stride, int octs_per_split) {
    __shared__ float red[gemv_fwd_max_waves(MT)][MT][8];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int half = lane & 1;
    const int sg = (segs.nseg > 1 && (int64_t)blockIdx.x >= segs.blk_start[1]) +
                   (segs.nseg > 2 && (int64_t)blockIdx.x >= segs.blk_start[2]);
    const WView& w = segs.w[sg];
    float* __restrict__ out = segs.out[sg];
    const int64_t out_ld = segs.out_ld[sg];
    const int64_t row_limit = segs.row_limit[sg];
    const int64_t R = (int64_t)blockIdx.x - segs.blk_start[sg];
    const int64_t kocts = w.k_pad >> 3;
    const int64_t o0 = (int64_t)blockIdx.y * octs_per_split;
    const int64_t o1 = min(o0 + (int64_t)octs_per_split, kocts);
    const uint8_t* rowbase = w.nib + 32 * (R * kocts) + 16 * half;
    const int64_t row0 = 8 * R + 4 * half;
    // every activation octet of the range is whole and 16-byte aligned: unguarded vector loads;
    // full: besides, every wave step covers 64 octets of the range (no dead octets to drop)
    const bool fast = x_vec && o1 * 8 <= w.K;
    const bool full = fast && (o1 - o0) % 64 == 0;

    float acc[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[m][r] = 0.0f;

    auto body = [&](auto fast_c, auto full_c) {
        constexpr bool kFast = decltype(fast_c)::value;
        constexpr bool kFull = decltype(full_c)::value;
        for (int64_t ob = o0 + (int64_t)wave * 64; ob < o1; ob += (int64_t)nw * 64) {
            u4 q[2];
            u4 sraw[2];               // fp16 scales: .xy; fp32 scales: all four
            u4 xr[2][MT];             // 8 activations (fp16/bf16), or the first 4 (fp32)
            f4 xr2[2][MT];            // fp32: the last 4
            bool live[2];
            // Every load of the iteration is issued before any of them is used; an octet past
            // the range reads the last valid one and is skipped below.
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t O = ob + 32 * j + (lane >> 1);
                live[j] = kFull || O < o1;
                const int64_t Oc = live[j] ? O : o1 - 1;
                const int64_t k0 = Oc * 8;
                q[j] = ldg16_stream(rowbase + 32 * Oc);
                // k0 < 2^31 (K <= 2^30): a 32-bit division, not the branchy 64-bit one
                const int64_t si = scale_index(w.g_pad, row0, (int64_t)((uint32_t)k0 / (uint32_t)w.gs));
                if constexpr (SF) {
                    const u2 v = *reinterpret_cast<const u2*>(static_cast<const uint16_t*>(w.scales) + si);
                    sraw[j] = u4{v.x, v.y, 0u, 0u};
                } else {
                    sraw[j] = *reinterpret_cast<const u4*>(static_cast<const float*>(w.scales) + si);
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const int64_t xb = m * w.K + k0;
                    if constexpr (kFast) {
                        if constexpr (XT == kF32) {
                            xr[j][m] = ldg16(static_cast<const float*>(x) + xb);
                            xr2[j][m] = *reinterpret_cast<const f4*>(static_cast<const float*>(x) + xb + 4);
                        } else {
                            xr[j][m] = ldg16(static_cast<const uint16_t*>(x) + xb);
                        }
                    } else if constexpr (XT == kF32) {
                        f4 a, b;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            a[e] = (k0 + e < w.K) ? static_cast<const float*>(x)[xb + e] : 0.0f;
                            b[e] = (k0 + 4 + e < w.K) ? static_cast<const float*>(x)[xb + 4 + e] : 0.0f;
                        }
                        xr[j][m] = bitcast<u4>(a);
                        xr2[j][m] = b;
                    } else {
                        uint32_t e[8];
#pragma unroll
                        for (int t = 0; t < 8; ++t)
                            e[t] = (k0 + t < w.K) ? static_cast<const uint16_t*>(x)[xb + t] : 0u;
                        xr[j][m] = u4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                      e[6] | (e[7] << 16)};
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);    // keep every load above ahead of every use below
            // a dead octet's terms are dropped by a select
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float sc[4];
                if constexpr (SF) {
                    sc[0] = f16_bits_to_f32((uint16_t)(sraw[j].x & 0xFFFFu));
                    sc[1] = f16_bits_to_f32((uint16_t)(sraw[j].x >> 16));
                    sc[2] = f16_bits_to_f32((uint16_t)(sraw[j].y & 0xFFFFu));
                    sc[3] = f16_bits_to_f32((uint16_t)(sraw[j].y >> 16));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sc[r] = bitcast<float>(sraw[j][r]);
                }
                const uint32_t wd[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
                if constexpr (XT == kF16) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        h2 c8[4];
#pragma unroll
                        for (int s = 0; s < 4; ++s) c8[s] = codes_minus8_f16(wd[r], s);
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            float t = 0.0f;
                            t = __builtin_amdgcn_fdot2(c8[0], bitcast<h2>(xr[j][m].x), t, false);
                            t = __builtin_amdgcn_fdot2(c8[1], bitcast<h2>(xr[j][m].y), t, false);
                            t = __builtin_amdgcn_fdot2(c8[2], bitcast<h2>(xr[j][m].z), t, false);
                            t = __builtin_amdgcn_fdot2(c8[3], bitcast<h2>(xr[j][m].w), t, false);
                            acc[m][r] = live[j] ? fmaf(t, sc[r], acc[m][r]) : acc[m][r];
                        }
                    }
                } else {
                    float xf[MT][8];
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        if constexpr (XT == kF32) {
                            const f4 a = bitcast<f4>(xr[j][m]);
                            const f4 b = xr2[j][m];
                            xf[m][0] = a.x; xf[m][1] = a.y; xf[m][2] = a.z; xf[m][3] = a.w;
                            xf[m][4] = b.x; xf[m][5] = b.y; xf[m][6] = b.z; xf[m][7] = b.w;
                        } else {
                            const uint32_t u[4] = {xr[j][m].x, xr[j][m].y, xr[j][m].z, xr[j][m].w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                xf[m][2 * e] = bitcast<float>(u[e] << 16);
                                xf[m][2 * e + 1] = bitcast<float>(u[e] & 0xFFFF0000u);
                            }
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float c[8];
                        word_codes_minus8_f32(wd[r], c);
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            float t = 0.0f;
#pragma unroll
                            for (int e = 0; e < 8; ++e) t = fmaf(xf[m][e], c[e], t);
                            acc[m][r] = live[j] ? fmaf(t, sc[r], acc[m][r]) : acc[m][r];
                        }
                    }
                }
            }
        }
    };
    if (full) body(std::true_type{}, std::true_type{});
    else if (fast) body(std::true_type{}, std::false_type{});
    else body(std::false_type{}, std::false_type{});

    // Sum over the 32 lanes holding the same four rows, then over the waves.
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc[m][r] = wave_sum_same_parity(acc[m][r]);
        }
    if (lane < 2) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][m][4 * lane + r] = acc[m][r];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < 8 * MT; t += blockDim.x) {
        const int m = t >> 3;
        const int r = t & 7;
        float v = 0.0f;
        for (int wv = 0; wv < nw; ++wv) v += red[wv][m][r];
        const int64_t n = 8 * R + r;
        if (n < row_limit) out[(int64_t)blockIdx.y * split_stride + m * out_ld + n] = v;
    }
}

// Weights of one row-octet decode launch (fields of one weight at index i).
struct RowSegs {
    const uint8_t* nib[3];
    const void* scales[3];
    float* out[3];
    int64_t N[3];
    int64_t n_octs[3];           // row-octets of the nibble plane (n_pad / 8)
    int64_t blk_start[4];        // first block of each weight; blk_start[nseg] = grid size
    int64_t g_pad, gs;           // shared: the weights share K and group size
    int nseg;
};

// Decode with one fp16 or bf16 activation row (M = 1; fp16: exact fp16 codes and dot2, bf16: x
// widened exactly to fp32 and fp32 FMA): P waves per row-octet each stream 1/P of its K
// (U x 64 k-octets in all), with every load (codes, scales, activations) issued before any use,
// sum their lanes with register-to-register cross-lane operations and, for P > 1, hand their row
// sums to the first wave through LDS (one barrier).  Taken when K = 512 U with U in 1..4, 8 or
// 16, x is 16-byte aligned and K is not split; lane l takes bytes [16 l, 16 l + 16) of each
// 32-micro-block run, as in gemv_fwd_kernel.  One launch serves up to three weights that share
// K, group size and scale dtype (the decode-shaped fused QKV): blocks [blk_start[i],
// blk_start[i + 1]) take weight i, with exactly the per-row work of a launch for weight i alone.
template <int SF, int U, int P, int XT>
__global__ __launch_bounds__(256) void gemv_fwd_row_kernel(RowSegs segs, const void* __restrict__ x) {
    static_assert(XT == kF16 || XT == kBF16, "16-bit activations");
    static_assert((P == 1 || P == 2 || P == 4) && (2 * U) % P == 0, "waves per row-octet");
    constexpr int I = 2 * U / P;                 // loads of each kind per lane
    __shared__ float part_s[4][8];               // P > 1: the row sums of waves kp > 0
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int sg = 0;
    while (sg + 1 < segs.nseg && (int64_t)blockIdx.x >= segs.blk_start[sg + 1]) ++sg;
    const uint8_t* const nib = segs.nib[sg];
    const void* const scales = segs.scales[sg];
    float* const out = segs.out[sg];
    const int64_t Rw = ((int64_t)blockIdx.x - segs.blk_start[sg]) * (4 / P) + wave / P;
    const int kp = wave % P;                     // which part of K the wave takes
    const bool live = Rw < segs.n_octs[sg];
    if constexpr (P == 1) {
        if (!live) return;                       // the whole wave
    }
    const int64_t R = live ? Rw : 0;             // a dead wave (P > 1) reads valid bytes it never uses
    const int half = lane & 1;
    constexpr int64_t kKocts = 64 * U;
    const uint8_t* rowbase = nib + 32 * (R * kKocts) + 16 * half;
    const int64_t row0 = 8 * R + 4 * half;
    u4 q[I], xr[I], sraw[I];
#pragma unroll
    for (int i = 0; i < I; ++i) {
        const int O = 32 * (I * kp + i) + (lane >> 1);
        q[i] = ldg16_stream(rowbase + 32 * O);
        const int64_t si = scale_index(segs.g_pad, row0, (int64_t)((uint32_t)(8 * O) / (uint32_t)segs.gs));
        if constexpr (SF) {
            const u2 v = *reinterpret_cast<const u2*>(static_cast<const uint16_t*>(scales) + si);
            sraw[i] = u4{v.x, v.y, 0u, 0u};
        } else {
            sraw[i] = *reinterpret_cast<const u4*>(static_cast<const float*>(scales) + si);
        }
        xr[i] = ldg16(static_cast<const uint16_t*>(x) + 8 * O);
    }
    __builtin_amdgcn_sched_barrier(0);          // keep every load above ahead of every use below
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < I; ++i) {
        float sc[4];
        if constexpr (SF) {
            sc[0] = f16_bits_to_f32((uint16_t)(sraw[i].x & 0xFFFFu));
            sc[1] = f16_bits_to_f32((uint16_t)(sraw[i].x >> 16));
            sc[2] = f16_bits_to_f32((uint16_t)(sraw[i].y & 0xFFFFu));
            sc[3] = f16_bits_to_f32((uint16_t)(sraw[i].y >> 16));
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[r] = bitcast<float>(sraw[i][r]);
        }
        const uint32_t wd[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
        if constexpr (XT == kF16) {
            // the nibble-pair mask and the fp16 1024 pair in registers: one v_and_or_b32 per pair
            uint32_t nib_mask = 0x000F000Fu, f16_1024 = 0x64006400u;
            asm volatile("" : "+s"(nib_mask));
            asm volatile("" : "+v"(f16_1024));
            const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
            auto pair = [&](uint32_t w, int e) {
                return bitcast<h2>(((w >> (4 * e)) & nib_mask) | f16_1024) - off;
            };
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float t = 0.0f;
                t = __builtin_amdgcn_fdot2(pair(wd[r], 0), bitcast<h2>(xr[i].x), t, false);
                t = __builtin_amdgcn_fdot2(pair(wd[r], 1), bitcast<h2>(xr[i].y), t, false);
                t = __builtin_amdgcn_fdot2(pair(wd[r], 2), bitcast<h2>(xr[i].z), t, false);
                t = __builtin_amdgcn_fdot2(pair(wd[r], 3), bitcast<h2>(xr[i].w), t, false);
                acc[r] = fmaf(t, sc[r], acc[r]);
            }
        } else {
            // bf16 x widened exactly to fp32 (the upper half of a word), exact fp32 codes, fp32 FMA
            const uint32_t xw[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
            float xf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xf[2 * e] = bitcast<float>(xw[e] << 16);
                xf[2 * e + 1] = bitcast<float>(xw[e] & 0xFFFF0000u);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float c[8];
                word_codes_minus8_f32(wd[r], c);
                float t = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) t = fmaf(xf[e], c[e], t);
                acc[r] = fmaf(t, sc[r], acc[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = wave_sum_same_parity(acc[r]);
    if constexpr (P > 1) {
        if (kp > 0 && lane < 2) {
#pragma unroll
            for (int r = 0; r < 4; ++r) part_s[wave][4 * lane + r] = acc[r];
        }
        __syncthreads();
        if (kp > 0 || !live) return;
#pragma unroll
        for (int p = 1; p < P; ++p)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += part_s[wave + p][4 * (lane & 1) + r];
    }
    if (lane < 2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = row0 + r;
            if (n < segs.N[sg]) out[n] = acc[r];
        }
    }
}

// Grid: (k_pad / 128, splits).  A block owns 128 columns of d_x; its waves take interleaved
// 32-row steps of the block's N range.  Per micro-block the output gradient is pre-scaled,
// d'[n] = d_out[m, n] * scale[g, n], and d_x[m, k] = sum_n d'[n] * (c[n, k] - 8).
template <int MT, int GT>
__global__ __launch_bounds__(256) void gemv_bwd_kernel(WView w, const void* __restrict__ d_out, int g_vec,
                                                       float* __restrict__ out, int64_t out_ld,
                                                       int64_t split_stride, int64_t col_limit,
                                                       int rsteps_per_split) {
    __shared__ float red[4][16][MT][8];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ro = lane >> 4;
    const int ko = lane & 15;
    const int64_t kocts = w.k_pad >> 3;
    const int64_t O = (int64_t)blockIdx.x * 16 + ko;
    const int64_t k0 = O * 8;
    const int64_t g = k0 / w.gs;
    const int total = (int)(w.n_pad >> 5);
    const int r0 = (int)blockIdx.y * rsteps_per_split;
    const int r1 = min(r0 + rsteps_per_split, total);

    float acc[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[m][j] = 0.0f;

    for (int rs = r0 + wave; rs < r1; rs += 4) {
        const int64_t R = (int64_t)rs * 4 + ro;
        const int64_t n0 = R * 8;
        uint32_t wd[8];
        load_micro_block(w.nib + 32 * (R * kocts + O), wd);
        float sc[8];
        load_scales8(w.scales, w.scale_f16, scale_index(w.g_pad, n0, g), sc);
        float dp[MT][8];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            load_act8<GT>(d_out, m * w.N + n0, n0, w.N, g_vec, dp[m]);
#pragma unroll
            for (int i = 0; i < 8; ++i) dp[m][i] *= sc[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float c[8];
            word_codes_minus8_f32(wd[i], c);
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[m][j] = fmaf(dp[m][i], c[j], acc[m][j]);
        }
    }

#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[m][j] = wave_sum_rows(acc[m][j]);
        }
    }
    if (ro == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < 8; ++j) red[wave][ko][m][j] = acc[m][j];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < 128 * MT; t += 256) {
        const int m = t >> 7;
        const int c = t & 127;
        const float v = (red[0][c >> 3][m][c & 7] + red[1][c >> 3][m][c & 7]) +
                        (red[2][c >> 3][m][c & 7] + red[3][c >> 3][m][c & 7]);
        const int64_t k = (int64_t)blockIdx.x * 128 + c;
        if (k < col_limit) out[(int64_t)blockIdx.y * split_stride + m * out_ld + k] = v;
    }
}

// Waves per block: one per 64 k-octets of the split, at most gemv_fwd_max_waves(M).  At K = 8192,
// N = 2048 the cap of 8 for M > 4 took 12.1 us at M = 8 against 33.8 with 16 waves and spills;
// M <= 4 keeps 16 (M = 1: 5.05 against 5.26 us with 8; cache-cold graph replay).
static int gemv_fwd_waves(const WView& w, int splits, int64_t M) {
    const int64_t octs = (w.k_pad / 8 + splits - 1) / splits;
    const int64_t nw = (octs + 63) / 64;
    const int64_t cap = gemv_fwd_max_waves(M);
    return (int)(nw > cap ? cap : (nw < 1 ? 1 : nw));
}

int gemv_fwd_splits(const WView& w, int64_t M) {
    (void)M;
    // One block per row-octet keeps every K step of those rows in one block (no reduction
    // launch).  Only very short N with long K splits K across blocks.
    const int64_t blocks = w.n_pad / 8;
    const int64_t octs = w.k_pad / 8;
    int64_t splits = 1;
    while (blocks * splits < 256 && octs / (splits * 2) >= 1024) splits *= 2;
    return (int)splits;
}

int gemv_bwd_splits(const WView& w, int64_t M) {
    (void)M;
    const int64_t blocks = w.k_pad / 128;
    const int64_t rsteps = w.n_pad / 32;
    int64_t splits = 1;
    while (blocks * splits < 512 && rsteps / (splits * 2) >= 4) splits *= 2;
    return (int)splits;
}

template <int XT, int SF>
static hipError_t gemv_fwd_dispatch(int64_t M, dim3 grid, dim3 block, hipStream_t s, const GemvSegs& segs,
                                    const void* x, int vec, int64_t stride, int per) {
    switch (M) {
#define Q4GSW_CASE(MT)                                                                                     \
    case MT:                                                                                               \
        hipLaunchKernelGGL((gemv_fwd_kernel<MT, XT, SF>), grid, block, 0, s, segs, x, vec, stride, per); \
        break;
        Q4GSW_CASE(1) Q4GSW_CASE(2) Q4GSW_CASE(3) Q4GSW_CASE(4)
        Q4GSW_CASE(5) Q4GSW_CASE(6) Q4GSW_CASE(7) Q4GSW_CASE(8)
#undef Q4GSW_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Waves per row-octet in the one-row decode: at K = 2048 two waves (half of K each) took 4.29 us
// per launch, one wave 4.43 and four 4.41 (cache-cold graph replay).  K = 4096 and 8192 take four
// waves (U / 2 loads per lane): N = 2048, K = 8192 took 4.39 us against 4.92 with
// gemv_fwd_kernel, and N = 14336, K = 4096 9.11 against 10.85.
constexpr int kRowP = 2;

template <int SF, int U, int XT>
static void launch_gemv_row_u(hipStream_t s, RowSegs segs, const void* x) {
    constexpr int P = U > 4 ? 4 : kRowP;
    int64_t b = 0;
    for (int i = 0; i < segs.nseg; ++i) {
        segs.blk_start[i] = b;
        b += (segs.n_octs[i] + 4 / P - 1) / (4 / P);
    }
    segs.blk_start[segs.nseg] = b;
    hipLaunchKernelGGL((gemv_fwd_row_kernel<SF, U, P, XT>), dim3((unsigned)b), dim3(256), 0, s, segs, x);
}

template <int SF, int XT>
static void launch_gemv_row(int u, hipStream_t s, const RowSegs& segs, const void* x) {
    switch (u) {
        case 1: launch_gemv_row_u<SF, 1, XT>(s, segs, x); break;
        case 2: launch_gemv_row_u<SF, 2, XT>(s, segs, x); break;
        case 3: launch_gemv_row_u<SF, 3, XT>(s, segs, x); break;
        case 4: launch_gemv_row_u<SF, 4, XT>(s, segs, x); break;
        case 8: launch_gemv_row_u<SF, 8, XT>(s, segs, x); break;
        default: launch_gemv_row_u<SF, 16, XT>(s, segs, x); break;
    }
}

bool gemv_row_eligible(const WView& w, const void* x, int x_dtype, int64_t M) {
    // bf16 x widens to fp32 and FMAs: at U = 16 that tail made the row kernel 4-5% slower than
    // gemv_fwd_kernel (N = 2048, K = 8192: 5.27 against 5.03 us), while U <= 8 gained 9-15%
    const int64_t u = w.k_pad / 512;
    return M == 1 && (x_dtype == kF16 || (x_dtype == kBF16 && u <= 8)) &&
           (reinterpret_cast<uintptr_t>(x) & 15u) == 0 && w.K == w.k_pad && w.k_pad % 512 == 0 &&
           (u <= 4 || u == 8 || u == 16) && gemv_fwd_splits(w, M) == 1;
}

hipError_t launch_gemv_fwd_row(const WView* w, float* const* out, int nseg, const void* x, int x_dtype,
                               hipStream_t s) {
    if (nseg < 1 || nseg > 3) return hipErrorInvalidValue;
    RowSegs segs{};
    segs.nseg = nseg;
    segs.g_pad = w[0].g_pad;
    segs.gs = w[0].gs;
    for (int i = 0; i < nseg; ++i) {
        if (w[i].k_pad != w[0].k_pad || w[i].gs != w[0].gs || w[i].scale_f16 != w[0].scale_f16)
            return hipErrorInvalidValue;
        segs.nib[i] = w[i].nib;
        segs.scales[i] = w[i].scales;
        segs.out[i] = out[i];
        segs.N[i] = w[i].N;
        segs.n_octs[i] = w[i].n_pad / 8;
    }
    const int u = (int)(w[0].k_pad / 512);
    if (x_dtype == kBF16) {
        if (w[0].scale_f16) launch_gemv_row<1, kBF16>(u, s, segs, x);
        else launch_gemv_row<0, kBF16>(u, s, segs, x);
    } else {
        if (w[0].scale_f16) launch_gemv_row<1, kF16>(u, s, segs, x);
        else launch_gemv_row<0, kF16>(u, s, segs, x);
    }
    return hipGetLastError();
}

// The streaming GEMV over nseg weights sharing K, group size and scale dtype; splits > 1 only with
// one weight (out is then the workspace [splits][M][n_pad]).
static hipError_t launch_gemv_fwd_segs(const WView* w, float* const* out, int nseg, const void* x, int x_dtype,
                                       int64_t M, int splits, hipStream_t s) {
    if (nseg < 1 || nseg > 3 || (nseg > 1 && splits != 1)) return hipErrorInvalidValue;
    GemvSegs segs{};
    segs.nseg = nseg;
    int64_t b = 0;
    for (int i = 0; i < nseg; ++i) {
        if (w[i].k_pad != w[0].k_pad || w[i].K != w[0].K || w[i].gs != w[0].gs || w[i].scale_f16 != w[0].scale_f16)
            return hipErrorInvalidValue;
        segs.w[i] = w[i];
        segs.out[i] = out[i];
        segs.out_ld[i] = splits == 1 ? w[i].N : w[i].n_pad;
        segs.row_limit[i] = splits == 1 ? w[i].N : w[i].n_pad;
        segs.blk_start[i] = b;
        b += w[i].n_pad / 8;
    }
    segs.blk_start[nseg] = b;
    const int64_t octs = w[0].k_pad / 8;
    const int per = (int)((octs + splits - 1) / splits);
    const int waves = gemv_fwd_waves(w[0], splits, M);
    const dim3 grid((unsigned)b, (unsigned)splits);
    const dim3 block((unsigned)(64 * waves));
    const int esize = x_dtype == kF32 ? 4 : 2;
    const int vec = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0) && ((w[0].K * esize) % 16 == 0);
    const int64_t stride = splits == 1 ? 0 : M * w[0].n_pad;
    if (w[0].scale_f16) {
        switch (x_dtype) {
            case kF32: return gemv_fwd_dispatch<kF32, 1>(M, grid, block, s, segs, x, vec, stride, per);
            case kF16: return gemv_fwd_dispatch<kF16, 1>(M, grid, block, s, segs, x, vec, stride, per);
            default: return gemv_fwd_dispatch<kBF16, 1>(M, grid, block, s, segs, x, vec, stride, per);
        }
    }
    switch (x_dtype) {
        case kF32: return gemv_fwd_dispatch<kF32, 0>(M, grid, block, s, segs, x, vec, stride, per);
        case kF16: return gemv_fwd_dispatch<kF16, 0>(M, grid, block, s, segs, x, vec, stride, per);
        default: return gemv_fwd_dispatch<kBF16, 0>(M, grid, block, s, segs, x, vec, stride, per);
    }
}

hipError_t launch_gemv_fwd(const WView& w, const void* x, int x_dtype, int64_t M, float* out, int splits,
                           hipStream_t s) {
    if (splits == 1 && gemv_row_eligible(w, x, x_dtype, M)) return launch_gemv_fwd_row(&w, &out, 1, x, x_dtype, s);
    return launch_gemv_fwd_segs(&w, &out, 1, x, x_dtype, M, splits, s);
}

hipError_t launch_gemv_fwd_multi(const WView* w, float* const* out, int nseg, const void* x, int x_dtype,
                                 int64_t M, hipStream_t s) {
    if (nseg >= 1 && gemv_row_eligible(w[0], x, x_dtype, M)) return launch_gemv_fwd_row(w, out, nseg, x, x_dtype, s);
    return launch_gemv_fwd_segs(w, out, nseg, x, x_dtype, M, 1, s);
}

template <int GT>
static hipError_t gemv_bwd_dispatch(int64_t M, dim3 grid, hipStream_t s, const WView& w, const void* g,
                                    int vec, float* out, int64_t ld, int64_t stride, int64_t limit, int per) {
    switch (M) {
#define Q4GSW_CASE(MT)                                                                                   \
    case MT:                                                                                             \
        hipLaunchKernelGGL((gemv_bwd_kernel<MT, GT>), grid, dim3(256), 0, s, w, g, vec, out, ld, stride, \
                           limit, per);                                                                  \
        break;
        Q4GSW_CASE(1) Q4GSW_CASE(2) Q4GSW_CASE(3) Q4GSW_CASE(4)
        Q4GSW_CASE(5) Q4GSW_CASE(6) Q4GSW_CASE(7) Q4GSW_CASE(8)
#undef Q4GSW_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_bwd(const WView& w, const void* d_out, int g_dtype, int64_t M, float* out, int splits,
                           hipStream_t s) {
    const int64_t rsteps = w.n_pad / 32;
    const int per = (int)((rsteps + splits - 1) / splits);
    const dim3 grid((unsigned)(w.k_pad / 128), (unsigned)splits);
    const int esize = g_dtype == kF32 ? 4 : 2;
    const int vec = ((reinterpret_cast<uintptr_t>(d_out) & 15u) == 0) && ((w.N * esize) % 16 == 0);
    const int64_t ld = splits == 1 ? w.K : w.k_pad;
    const int64_t stride = splits == 1 ? 0 : M * w.k_pad;
    const int64_t limit = splits == 1 ? w.K : w.k_pad;
    switch (g_dtype) {
        case kF32: return gemv_bwd_dispatch<kF32>(M, grid, s, w, d_out, vec, out, ld, stride, limit, per);
        case kF16: return gemv_bwd_dispatch<kF16>(M, grid, s, w, d_out, vec, out, ld, stride, limit, per);
        default: return gemv_bwd_dispatch<kBF16>(M, grid, s, w, d_out, vec, out, ld, stride, limit, per);
    }
}

}  // namespace q4gsw
