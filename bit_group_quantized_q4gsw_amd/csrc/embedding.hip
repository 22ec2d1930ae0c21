// Embedding row gather from a packed q4gsw weight: out[t, k] = dequant(W[ids[t], k]).
//
// embedding_q4gsw is one of the ops of the Gemma 4 ExecuTorch export (a maintainer comment on
// the react-native-executorch issue about upstreaming the Gemma 4 Vulkan support lists its fp16
// bugs among the exporter changes).  The WebGPU pull request that keeps the Q4 embedding's
// shader controls across resize gives it an is_linear_weight flag: the table may share the
// nibble layout of a linear weight.  Here the table is a packed linear weight [N rows, K
// columns] (one buffer for a tied embedding and output projection), and row t of the output is
// row ids[t] of dequant(W).  The pages do not say what an id outside [0, N) gives: here a row of
// zeros, and the table is not read for it.
//
// Work unit: one lane per (token, k-octet).  A lane reads the 4-byte word of row n at its octet
// and the octet's scale, then writes 8 fp32 values.  Consecutive lanes take consecutive octets of
// one token, so a wave's stores cover 2 KB of one output row; the reads of a wave touch one word
// in each of 64 micro-blocks (the layout interleaves 8 rows per 32 bytes, so a gather of one row
// pulls whole sectors holding 7 other rows).  The output write, 4 bytes per element against half a
// byte of codes, is the larger stream.
#include "device.h"
#include "internal.h"

namespace q4gsw {

// 64 lanes per block: 512 ids of 2048 columns took 3.03 us per launch against 3.06 with 128 and
// 3.11 with 256 lanes, and two octets per lane was slower (3.23 us; cache-cold graph replay).
constexpr int kEmbThreads = 64;

struct EmbArgs {
    const uint8_t* nib;
    const void* scales;
    const int64_t* ids;
    float* out;
    int64_t N, K, gs, k_pad, g_pad, T;
    int64_t octs;             // ceil(K / 8)
    uint32_t blocks_per_row;  // ceil(octs / kEmbThreads)
    int scale_f16;
};

// VEC: K % 8 == 0 and out 16-byte aligned (two 16-byte stores per lane).
// G8: group_size % 8 == 0 (one scale per octet).
template <bool VEC, bool G8>
__global__ __launch_bounds__(kEmbThreads) void embedding_kernel(EmbArgs a) {
    const uint32_t row_block = blockIdx.x / a.blocks_per_row;
    const int64_t t = row_block;
    const int64_t o = (int64_t)(blockIdx.x - row_block * a.blocks_per_row) * kEmbThreads + threadIdx.x;
    if (o >= a.octs) return;
    const int64_t n = a.ids[t];
    const bool valid = n >= 0 && n < a.N;
    // both loads are issued before any use; a lane of an id outside [0, N) reads nothing and takes
    // the word of eight code-8 nibbles (value 0)
    const uint32_t word = valid ? *reinterpret_cast<const uint32_t*>(a.nib + word_offset(a.k_pad, n, o)) : 0x88888888u;
    const float s8 = (valid && G8) ? load_scale(a.scales, a.scale_f16, scale_index(a.g_pad, n, (8 * o) / a.gs)) : 0.0f;
    float c[8];
    word_codes_minus8_f32(word, c);
    float v[8];
    if (G8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = c[j] * s8;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t k = 8 * o + j;
            // columns K..k_pad-1 exist in the packed buffer (code 8, scale 0) but are not written
            v[j] = (valid && k < a.K) ? c[j] * load_scale(a.scales, a.scale_f16, scale_index(a.g_pad, n, k / a.gs))
                                      : 0.0f;
        }
    }
    float* dst = a.out + t * a.K + 8 * o;
    if (VEC) {
        reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (8 * o + j < a.K) dst[j] = v[j];
    }
}

uint64_t embedding_blocks(int64_t T, int64_t K) {
    const int64_t octs = (K + 7) / 8;
    return (uint64_t)T * (uint64_t)((octs + kEmbThreads - 1) / kEmbThreads);
}

hipError_t launch_embedding(const WView& w, const int64_t* ids, int64_t T, float* out, hipStream_t s) {
    EmbArgs a;
    a.nib = w.nib;
    a.scales = w.scales;
    a.ids = ids;
    a.out = out;
    a.N = w.N;
    a.K = w.K;
    a.gs = w.gs;
    a.k_pad = w.k_pad;
    a.g_pad = w.g_pad;
    a.T = T;
    a.octs = (w.K + 7) / 8;
    a.blocks_per_row = (uint32_t)((a.octs + kEmbThreads - 1) / kEmbThreads);
    a.scale_f16 = w.scale_f16;
    const uint64_t blocks = embedding_blocks(T, w.K);
    if (blocks == 0 || blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const bool vec = w.K % 8 == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0;
    const bool g8 = w.gs % 8 == 0;
    const dim3 grid((unsigned)blocks), block(kEmbThreads);
    if (vec && g8)
        hipLaunchKernelGGL((embedding_kernel<true, true>), grid, block, 0, s, a);
    else if (vec)
        hipLaunchKernelGGL((embedding_kernel<true, false>), grid, block, 0, s, a);
    else if (g8)
        hipLaunchKernelGGL((embedding_kernel<false, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((embedding_kernel<false, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace q4gsw
