// linear_dq8ca_q4gsw on gfx950: the q4gsw forward with activations quantised to int8 per row
// on the fly, then an int8 x int4 MFMA GEMM.
//
// The pages name the op (the shader changes of linear_q4gsw / linear_dq8ca_q4gsw in the "Suggested
// split" of the react-native-executorch Gemma 4 Vulkan issue) and nothing more.  Reading: "dq8" a
// dynamic int8 activation, "ca" per channel of the activation (per row / token), asymmetric, with
// zero exact.  For each row, every step in fp32 as written (rint: round half to even):
//   lo = min(0, min x), hi = max(0, max x), scale = (hi - lo) / 255 (at least the smallest normal
//   fp32), inv = 1 / scale, zp = clamp(-128 - rint(lo * inv)), q = clamp(rint(x * inv) + zp),
// both clamps to [-128, 127]; the row stands for scale * (q - zp), and
//   y[m, n] = scale[m] * sum_g s[g, n] * T_g[m, n],   T_g = sum_{k in group g} (q - zp) (code - 8).
//
// Quantisation (dq8ca_quant_kernel): one block per row, min / max reduction, the fp32 steps above
// (IEEE division and rint, as in the definition), then the codes.  For the GEMM the codes of each
// row are written k_pad long (zero padding) with every k-octet's bytes in the order in which the
// B operand below yields the nibbles of a packed word, k-offsets 0, 4, 1, 5, 2, 6, 3, 7, so A
// and B bytes meet the same k in the dot product.
//
// GEMM (dq8ca_gemm_kernel): v_mfma_i32_32x32x32_i8, exact int32 accumulation.
//   * block = 8 waves side by side in N, each 128 (M) x 32 (N) = four 32x32 tiles; a 64-column
//     K chunk is two MFMA steps;
//   * every global read is an LDS-DMA into a 3-stage ring, 2 chunks ahead: the block's 128 x 64
//     int8 activation tile (one 1 KB DMA per wave; 16-byte slots swizzled by (row >> 2) & 3 so an
//     A-fragment read phase covers all banks), each wave's 1 KB of codes (row-octet runs rotated
//     by 2R 32-byte blocks), and the block's scales of the chunk's groups (wave 0);
//   * B = code - 8 as int8, built per packed word with a mask, an add of 0x78 and an xor of 0x80
//     per byte (no carries: every byte stays below 0x88);
//   * zero point: q = (q - zp) + zp, so T_g = sum q (code - 8) + (-zp) W_g[n] with
//     W_g[n] = sum_{k in g} (code - 8), summed from the same B bytes with v_dot4 against ones:
//     the correction is exact in int32 before any rounding;
//   * at the end of each group (or of the split) T_g is converted to fp32 (exact: |T_g| < 2^24
//     for gs <= 8192) and accumulated as fp32 fma(T_g, s[g, n], total); the row scale multiplies
//     the total in the epilogue.  Error: at most (groups + 2) fp32 roundings of the result;
//   * K splits across blocks as in the fp16 forward: fp32 partials in the 32x32 fragment order,
//     summed in split order by the reduction kernel.
#include "device.h"
#include "internal.h"

#include <float.h>

namespace q4gsw {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kWN = 32;
constexpr int kBN = kWaves * kWN;    // block columns
constexpr int kBM = 128;             // block rows
constexpr int kCK = 64;              // K columns per chunk
constexpr int kRow = 64;             // bytes of one activation row of a chunk
constexpr int kABytes = kBM * kRow;  // 8 KB
constexpr int kCodeBytes = 1024;     // one wave's codes of a chunk

// k-offset held by byte position p of a GEMM-layout octet
__device__ constexpr int kPerm[8] = {0, 4, 1, 5, 2, 6, 3, 7};

// ---------------------------------------------------------------------------------------------
// The row's range, scale and zero point from its min / max (every step in fp32 as defined).
struct RowQuant {
    float s, inv;
    int z;
    __device__ int operator()(float v) const {
        const int t = (int)rintf(v * inv) + z;
        return t < -128 ? -128 : (t > 127 ? 127 : t);
    }
};

__device__ __forceinline__ RowQuant row_quant(float lo, float hi, float (*red)[4]) {
    const int tid = threadIdx.x;
    for (int off = 32; off >= 1; off >>= 1) {
        const float l2 = __shfl_xor(lo, off);
        const float h2 = __shfl_xor(hi, off);
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
    }
    if ((tid & 63) == 0) {
        red[0][tid >> 6] = lo;
        red[1][tid >> 6] = hi;
    }
    __syncthreads();
    lo = red[0][0];
    hi = red[1][0];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        lo = red[0][i] < lo ? red[0][i] : lo;
        hi = red[1][i] > hi ? red[1][i] : hi;
    }
    RowQuant r;
    r.s = (hi - lo) / 255.0f;
    if (r.s < FLT_MIN) r.s = FLT_MIN;
    r.inv = 1.0f / r.s;
    const int z = -128 - (int)rintf(lo * r.inv);
    r.z = z < -128 ? -128 : (z > 127 ? 127 : z);
    return r;
}

// one k-octet of a row: 8 values from one (16-bit types) or two (fp32) 16-byte loads
template <int XT>
__device__ __forceinline__ void load_octet(const void* x, int64_t e, float (&v)[8]) {
    if constexpr (XT == kF32) {
        const f4 a = bitcast<f4>(ldg16(static_cast<const float*>(x) + e));
        const f4 b = bitcast<f4>(ldg16(static_cast<const float*>(x) + e + 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = a[i];
            v[4 + i] = b[i];
        }
    } else {
        const u4 a = ldg16(static_cast<const uint16_t*>(x) + e);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint16_t l = (uint16_t)(a[i] & 0xFFFFu), h = (uint16_t)(a[i] >> 16);
            v[2 * i] = XT == kF16 ? f16_bits_to_f32(l) : bf16_bits_to_f32(l);
            v[2 * i + 1] = XT == kF16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
        }
    }
}

// XT: activation dtype.  GEMM: write the GEMM layout (rows of ld bytes, permuted octets, zero
// padding) and -zp; else the natural [M, K] codes and zp.  VEC: K % 8 == 0 and x 16-byte aligned,
// so every octet is read with 16-byte loads; the min / max pass keeps kOcts octets per thread in
// flight.  One block of 256 threads per row.
constexpr int kOcts = 4;

template <int XT, bool GEMM, bool VEC>
__global__ __launch_bounds__(256) void dq8ca_quant_kernel(const void* __restrict__ x, int64_t K, int64_t ld,
                                                          int8_t* __restrict__ q, float* __restrict__ scale,
                                                          int32_t* __restrict__ zpo) {
    __shared__ float red[2][4];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    float lo = 0.0f, hi = 0.0f;
    // a row of at most 256 kOcts octets (K <= 8192) is read once: the min / max pass leaves each
    // thread's octets in v for the codes
    float v[kOcts][8];
    if constexpr (VEC) {
        const int64_t octs = K >> 3;
        for (int64_t o0 = 0; o0 < octs; o0 += 256 * kOcts) {
#pragma unroll
            for (int i = 0; i < kOcts; ++i) {
                const int64_t o = o0 + tid + 256 * i;
                if (o < octs) load_octet<XT>(x, m * K + 8 * o, v[i]);
            }
#pragma unroll
            for (int i = 0; i < kOcts; ++i) {
                if (o0 + tid + 256 * i >= octs) continue;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    lo = v[i][e] < lo ? v[i][e] : lo;
                    hi = v[i][e] > hi ? v[i][e] : hi;
                }
            }
        }
    } else {
        for (int64_t k = tid; k < K; k += 256) {
            const float e = load_elem<XT>(x, m * K + k);
            lo = e < lo ? e : lo;
            hi = e > hi ? e : hi;
        }
    }
    const RowQuant rq = row_quant(lo, hi, red);
    if constexpr (VEC) {
        // 8 codes per octet, one 8-byte store; longer rows read the row again (now in L2)
        const int64_t octs = K >> 3;
        if (octs <= 256 * kOcts) {
#pragma unroll
            for (int i = 0; i < kOcts; ++i) {
                const int64_t o = tid + 256 * i;
                if (o >= octs) continue;
                uint32_t wd[2] = {0u, 0u};
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const int k = GEMM ? kPerm[p] : p;
                    wd[p >> 2] |= (uint32_t)(rq(v[i][k]) & 0xFF) << (8 * (p & 3));
                }
                *reinterpret_cast<u2*>(q + m * ld + 8 * o) = u2{wd[0], wd[1]};
            }
        } else {
            for (int64_t o = tid; o < octs; o += 256) {
                float w[8];
                load_octet<XT>(x, m * K + 8 * o, w);
                uint32_t wd[2] = {0u, 0u};
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const int k = GEMM ? kPerm[p] : p;
                    wd[p >> 2] |= (uint32_t)(rq(w[k]) & 0xFF) << (8 * (p & 3));
                }
                *reinterpret_cast<u2*>(q + m * ld + 8 * o) = u2{wd[0], wd[1]};
            }
        }
        if constexpr (GEMM)
            for (int64_t o = octs + tid; o < ld / 8; o += 256) *reinterpret_cast<u2*>(q + m * ld + 8 * o) = u2{0u, 0u};
    } else if constexpr (GEMM) {
        for (int64_t o = tid; o < ld / 8; o += 256) {
            uint32_t wd[2] = {0u, 0u};
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int64_t k = 8 * o + kPerm[p];
                const int t = k < K ? rq(load_elem<XT>(x, m * K + k)) : 0;
                wd[p >> 2] |= (uint32_t)(t & 0xFF) << (8 * (p & 3));
            }
            *reinterpret_cast<u2*>(q + m * ld + 8 * o) = u2{wd[0], wd[1]};
        }
    } else {
        for (int64_t k = tid; k < K; k += 256) q[m * K + k] = (int8_t)rq(load_elem<XT>(x, m * K + k));
    }
    if (tid == 0) {
        scale[m] = rq.s;
        zpo[m] = GEMM ? -rq.z : rq.z;
    }
}

// ---------------------------------------------------------------------------------------------
// SF: 1 = fp16 scales.  SPC: scale groups per 64-column chunk (1: gs % 64 == 0, 2: gs == 32,
// where every 32-column MFMA step is one group).
template <int SF, int SPC>
__global__ __launch_bounds__(512, 1) void dq8ca_gemm_kernel(WView w, const int8_t* __restrict__ aq,
                                                            const float* __restrict__ rs, const int32_t* __restrict__ nzp,
                                                            int64_t M, float* __restrict__ out, int64_t out_ld,
                                                            int64_t split_stride, int chunks_per_split, int splits,
                                                            int mtiles) {
    constexpr int kStages = 3;
    constexpr int kSDma = SF ? 1 : SPC;                       // wave 0's scale DMAs per chunk
    constexpr int kAOff = 0, kBOff = kABytes, kSOff = kBOff + kWaves * kCodeBytes;
    constexpr int kStage = kSOff + 1024 * kSDma;
    constexpr int kDma = 2;                                    // DMAs of every wave per chunk
    // one LDS array for everything: with several, the compiler gives each its own alias scope and
    // then waits for every LDS-DMA in flight before any read of the ring, which drains the
    // prefetch each chunk
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStage + 8 * kBM];
    int32_t* const s_nzp = reinterpret_cast<int32_t*>(smem + kStages * kStage);
    float* const s_rs = reinterpret_cast<float*>(smem + kStages * kStage + 4 * kBM);
    lds_u8* const sm_l = (lds_u8*)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;
    const int h = lane >> 5;

    const int64_t bid = blockIdx.x;
    const int z = (int)(bid % splits);
    const int64_t rest = bid / splits;
    const int64_t mb = rest % mtiles;
    const int64_t tile = rest / mtiles;
    const int64_t n0 = tile * kBN + (int64_t)wave * kWN;
    const bool wave_active = n0 < w.n_pad;
    const int64_t nw = wave_active ? n0 : 0;
    const int64_t m0 = mb * kBM;
    const int64_t kp = w.k_pad;
    const int64_t kocts = kp >> 3;
    const int64_t n_chunks = kp / kCK;
    const int64_t c_begin = (int64_t)z * chunks_per_split;
    const int64_t c_end = min(c_begin + (int64_t)chunks_per_split, n_chunks);

    if (tid < kBM) {
        const int64_t m = m0 + tid;
        s_nzp[tid] = m < M ? nzp[m] : 0;
        s_rs[tid] = m < M ? rs[m] : 0.0f;
    }

    // ---- DMA sources ----
    // activations: wave w's DMA covers block rows 16 w .. 16 w + 15; lane l fills row 16 w + l / 4,
    // physical slot l % 4, which holds logical slot (l % 4) ^ ((row >> 2) & 3)
    const int arow = 16 * wave + (lane >> 2);
    const int64_t am = min(m0 + arow, M - 1);          // rows past M only feed discarded outputs
    const int8_t* asrc = aq + am * kp + 16 * ((lane & 3) ^ ((arow >> 2) & 3));
    // codes: lane l fills LDS bytes 16 l = row-octet R = l >> 4, rotated block slot p = (l & 15) >> 1,
    // half l & 1, which holds k-octet (p - 2R) & 7 of the chunk
    const uint8_t* csrc;
    {
        const int R = lane >> 4;
        const int o = (((lane & 15) >> 1) - 2 * R) & 7;
        csrc = w.nib + 32 * (((nw >> 3) + R) * kocts + o) + 16 * (lane & 1);
    }
    const uint8_t* sptr = static_cast<const uint8_t*>(w.scales);
    const int64_t boct = tile * (kBN / 8);
    const int64_t n_octs = w.n_pad / 8;
    auto issue = [&](int64_t c, int st) {
        lds_u8* base = sm_l + st * kStage;
        dma16(asrc + kCK * c, base + kAOff + kRow * 16 * wave);
        dma16(csrc + 256 * c, base + kBOff + wave * kCodeBytes);
        if (wave == 0) {
            const uint32_t kc = (uint32_t)(c * kCK);
#pragma unroll
            for (int i = 0; i < kSDma; ++i) {
                // lane -> (row-octet o of the block, group slot q, 16-byte half of an fp32 run);
                // fp16 with one slot: lanes 32..63 repeat lanes 0..31
                int o, qq, half;
                if constexpr (SF) {
                    o = (lane / SPC) & 31;
                    qq = lane % SPC;
                    half = 0;
                } else {
                    const int P = 32 * i + (lane >> 1);
                    o = P / SPC;
                    qq = P % SPC;
                    half = lane & 1;
                }
                const int64_t g = (int64_t)((kc + 32u * (uint32_t)qq) / (uint32_t)w.gs);
                const int64_t oct = min(boct + o, n_octs - 1);
                const int64_t idx = (oct * w.g_pad + g) * 8;
                dma16(SF ? sptr + 2 * idx : sptr + 4 * idx + 16 * half, base + kSOff + 1024 * i);
            }
        }
    };

    // ---- accumulators ----
    v16i acc[4];
    f32x16 tot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[i][r] = 0;
            tot[i][r] = 0.f;
        }
    int wpart = 0;                       // sum of this lane's codes - 8 in the open group (its k half)
    const int srl = 32 * wave + j;       // the lane's column inside the block
    const int Rj = j >> 3;

    // total += T_g * s (T_g = acc + (-zp) W_g, exact in int32); then the group's sums restart
    auto close_group = [&](const uint8_t* S, int qslot) {
        const uint32_t wp = (uint32_t)wpart;
        const auto sw = __builtin_amdgcn_permlane32_swap(wp, wp, false, false);
        const int Wg = (int)sw[0] + (int)sw[1];
        float sg;
        const int so = (SF ? 16 : 32) * (SPC * (srl >> 3) + qslot) + (SF ? 2 : 4) * (srl & 7);
        if constexpr (SF) sg = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(S + so));
        else sg = *reinterpret_cast<const float*>(S + so);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const v4i nz = *reinterpret_cast<const v4i*>(&s_nzp[32 * mi + 8 * r4 + 4 * h]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * r4 + e;
                    const int T = acc[mi][r] + __mul24(nz[e], Wg);
                    tot[mi][r] = fmaf((float)T, sg, tot[mi][r]);
                }
            }
        }
        wpart = 0;
    };

    // one 32-column MFMA step t of the chunk in stage st; the first step of a group (fresh)
    // starts its sums from zero through the MFMA's accumulator operand
    const v16i zero16 = {};
    auto step = [&](int st, int t, auto fresh) {
        const uint8_t* Ab = smem + st * kStage + kAOff;
        const uint8_t* Bb = smem + st * kStage + kBOff + wave * kCodeBytes;
        // B: the two code words of k-octets 4t + 2h and 4t + 2h + 1 of the lane's column
        uint32_t wd[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int O = 4 * t + 2 * h + u;
            wd[u] = *reinterpret_cast<const uint32_t*>(Bb + 256 * Rj + 32 * ((O + 2 * Rj) & 7) + 4 * (j & 7));
        }
        v4i b;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            b[2 * u] = (int)(((wd[u] & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
            b[2 * u + 1] = (int)((((wd[u] >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) wpart = __builtin_amdgcn_sdot4(b[e], 0x01010101, wpart, false);
        const int slot = 2 * t + h;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int row = 32 * mi + j;
            const v4i a = *reinterpret_cast<const v4i*>(Ab + kRow * row + 16 * (slot ^ ((row >> 2) & 3)));
            acc[mi] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, decltype(fresh)::value ? zero16 : acc[mi], 0, 0, 0);
        }
    };

    // ---- pipeline: DMAs 2 chunks ahead into a 3-stage ring ----
    if (c_begin < c_end) issue(c_begin, 0);
    if (c_begin + 1 < c_end) issue(c_begin + 1, 1);
    int st = 0;
    // MFMA steps (32 columns each) per scale group and, counting down, those left in the open one
    const int spg = (int)(w.gs / 32);
    int left = spg - (int)((2 * c_begin) % spg);
    bool fresh = true;                   // the next step opens a group
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int st_next = st == 2 ? 0 : st + 1;
        const int st_prev = st == 0 ? 2 : st - 1;
        if (c + 1 < c_end) {
            if (wave == 0) wait_loads_barrier<kDma + kSDma>();
            else wait_loads_barrier<kDma>();
        } else {
            wait_loads_barrier<0>();
        }
        if (c + 2 < c_end) issue(c + 2, st_prev);
        const uint8_t* S = smem + st * kStage + kSOff;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (SPC == 2 || fresh) step(st, t, std::true_type{});
            else step(st, t, std::false_type{});
            // a group closes at its last step, and the open group at the split's last step
            bool close = true;
            if constexpr (SPC == 1) {
                close = --left == 0 || (t == 1 && c + 1 == c_end);
                if (left == 0) left = spg;
            }
            if (close) close_group(S, SPC == 2 ? t : 0);
            fresh = close;
        }
        st = st_next;
    }

    // ---- epilogue: lane holds D[8 (r/4) + 4 h + r%4][j] of each 32x32 tile ----
    if (!wave_active) return;
    if (split_stride) {
        float* plane = out + (int64_t)z * split_stride;
        const int64_t tn = n0 / 32;
        const int64_t ntn = out_ld / 32;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int64_t tm = m0 / 32 + mi;
            if (32 * tm >= M) break;
            float* tp = plane + (tm * ntn + tn) * 1024 + 4 * lane;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f4 sc = *reinterpret_cast<const f4*>(&s_rs[32 * mi + 8 * r4 + 4 * h]);
                __builtin_nontemporal_store(f4{sc[0] * tot[mi][4 * r4], sc[1] * tot[mi][4 * r4 + 1],
                                               sc[2] * tot[mi][4 * r4 + 2], sc[3] * tot[mi][4 * r4 + 3]},
                                            reinterpret_cast<f4*>(tp + 256 * r4));
            }
        }
        return;
    }
    const int64_t n = n0 + j;
    if (n >= w.N) return;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 32 * mi + 8 * (r >> 2) + 4 * h + (r & 3);
            const int64_t m = m0 + row;
            if (m < M) out[m * out_ld + n] = s_rs[row] * tot[mi][r];
        }
    }
}

}  // namespace

bool dq8ca_supported(const WView& w) { return w.gs % 64 == 0 || w.gs == 32; }

uint64_t dq8ca_blocks_limit() { return uint64_t(1) << 24; }

static int64_t dq8ca_codes_bytes(int64_t M, int64_t kp) { return round_up(M * kp, 256); }
static int64_t dq8ca_rows_bytes(int64_t M) { return round_up(M * 4, 256); }

Dq8caPlan plan_dq8ca(const WView& w, int64_t M, int force_splits) {
    Dq8caPlan p{};
    const int64_t tiles = (w.n_pad + kBN - 1) / kBN;
    const int64_t blocks = tiles * ((M + kBM - 1) / kBM);
    const int64_t n_chunks = w.k_pad / kCK;
    p.splits = pick_gemm_splits(blocks, n_chunks, M, w.n_pad, 256, 1.5, nullptr, force_splits);
    p.ws_bytes = dq8ca_codes_bytes(M, w.k_pad) + 2 * dq8ca_rows_bytes(M) +
                 (p.splits > 1 ? (int64_t)p.splits * frag_plane_floats(M, w.n_pad) * 4 : 0);
    return p;
}

template <bool GEMM>
static hipError_t launch_quant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ld, int8_t* q, float* scale,
                               int32_t* zp, hipStream_t s) {
    if (M > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)M);
    const bool vec = K % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0 &&
                     (GEMM || (reinterpret_cast<uintptr_t>(q) & 7u) == 0);
#define Q4GSW_DQ8CA_QUANT(XT)                                                                             \
    if (vec) hipLaunchKernelGGL((dq8ca_quant_kernel<XT, GEMM, true>), grid, dim3(256), 0, s, x, K, ld, q, scale, zp); \
    else hipLaunchKernelGGL((dq8ca_quant_kernel<XT, GEMM, false>), grid, dim3(256), 0, s, x, K, ld, q, scale, zp);
    switch (x_dtype) {
        case kF32: Q4GSW_DQ8CA_QUANT(kF32) break;
        case kF16: Q4GSW_DQ8CA_QUANT(kF16) break;
        default: Q4GSW_DQ8CA_QUANT(kBF16) break;
    }
#undef Q4GSW_DQ8CA_QUANT
    return hipGetLastError();
}

hipError_t launch_dq8ca_quantize(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q, float* scale,
                                 int32_t* zp, hipStream_t s) {
    return launch_quant<false>(x, x_dtype, M, K, K, q, scale, zp, s);
}

hipError_t launch_dq8ca(const WView& w, const void* x, int x_dtype, int64_t M, float* y, const Dq8caPlan& plan,
                        void* ws, hipStream_t s) {
    if (!dq8ca_supported(w) || M > 0x7fffffff) return hipErrorInvalidValue;
    uint8_t* base = static_cast<uint8_t*>(ws);
    int8_t* aq = reinterpret_cast<int8_t*>(base);
    float* rs = reinterpret_cast<float*>(base + dq8ca_codes_bytes(M, w.k_pad));
    int32_t* nzp = reinterpret_cast<int32_t*>(base + dq8ca_codes_bytes(M, w.k_pad) + dq8ca_rows_bytes(M));
    float* part = reinterpret_cast<float*>(base + dq8ca_codes_bytes(M, w.k_pad) + 2 * dq8ca_rows_bytes(M));
    hipError_t e = launch_quant<true>(x, x_dtype, M, w.K, w.k_pad, aq, rs, nzp, s);
    if (e != hipSuccess) return e;
    const int64_t tiles = (w.n_pad + kBN - 1) / kBN;
    const int64_t mtiles = (M + kBM - 1) / kBM;
    const int64_t n_chunks = w.k_pad / kCK;
    const int per = (int)((n_chunks + plan.splits - 1) / plan.splits);
    const int64_t blocks = tiles * mtiles * plan.splits;
    if (blocks > (int64_t)dq8ca_blocks_limit()) return hipErrorInvalidConfiguration;
    float* out = plan.splits == 1 ? y : part;
    const int64_t ld = plan.splits == 1 ? w.N : w.n_pad;
    const int64_t stride = plan.splits == 1 ? 0 : frag_plane_floats(M, w.n_pad);
    const int sp = plan.splits, mt = (int)mtiles;
    const dim3 grid((unsigned)blocks);
    const bool two = w.gs == 32;
    if (w.scale_f16) {
        if (two) hipLaunchKernelGGL((dq8ca_gemm_kernel<1, 2>), grid, dim3(512), 0, s, w, aq, rs, nzp, M, out, ld, stride, per, sp, mt);
        else hipLaunchKernelGGL((dq8ca_gemm_kernel<1, 1>), grid, dim3(512), 0, s, w, aq, rs, nzp, M, out, ld, stride, per, sp, mt);
    } else {
        if (two) hipLaunchKernelGGL((dq8ca_gemm_kernel<0, 2>), grid, dim3(512), 0, s, w, aq, rs, nzp, M, out, ld, stride, per, sp, mt);
        else hipLaunchKernelGGL((dq8ca_gemm_kernel<0, 1>), grid, dim3(512), 0, s, w, aq, rs, nzp, M, out, ld, stride, per, sp, mt);
    }
    e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const float* ys[1] = {y};
    const int64_t yld[1] = {w.N}, off[1] = {0}, cols[1] = {w.N};
    return launch_reduce_frags(part, plan.splits, M, w.n_pad, ys, yld, off, cols, 1, 0, s);
}

}  // namespace q4gsw
