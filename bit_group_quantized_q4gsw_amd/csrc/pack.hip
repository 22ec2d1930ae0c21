// One-time repack of q4gsw codes and scales into the gfx950 layout, and its inverse.
//
// The pages prepack the weight and scales once and reuse that buffer in forward
// and backward (Vulkan q4gsw-backward PR body, "Key changes"; WebGPU BK64 QKV PR
// body).  The byte layout itself is this library's (see layout.h).
#include "device.h"
#include "internal.h"

namespace q4gsw {

__global__ void clear_header_kernel(uint32_t* hdr) { hdr[threadIdx.x] = 0u; }

// One thread per 32-bit output word; consecutive threads write consecutive words.
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes, int64_t N,
                                                         int64_t K, int64_t n_pad, int64_t k_pad,
                                                         uint32_t* __restrict__ nib,
                                                         uint32_t* __restrict__ hdr) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t kocts = k_pad >> 3;
    if (t >= n_pad * kocts) return;
    const int64_t i = t & 7;
    const int64_t blk = t >> 3;
    const int64_t n = (blk / kocts) * 8 + i;
    const int64_t o = blk % kocts;
    uint32_t word = 0u;
    uint32_t bad = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t k = o * 8 + j;
        uint32_t c = 8u;
        if (n < N && k < K) {
            c = codes[n * K + k];
            bad |= (c > 15u);
            c &= 15u;
        }
        word |= c << (4 * nib_pos(j));
    }
    nib[t] = word;
    if (bad) hdr[kHdrBadCode] = 1u;          // every writer stores the same value
}

// One thread per stored scale, in plane order [n / 8][group][n % 8]; padding gets 0.  For
// fp16 scales also checks that (code - 8) * s stays a finite normal fp16 for every code.
__global__ __launch_bounds__(256) void pack_scales_kernel(const void* __restrict__ src, int scale_f16,
                                                          int64_t N, int64_t G, int64_t n_pad,
                                                          int64_t g_pad, void* __restrict__ dst,
                                                          uint32_t* __restrict__ hdr) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= g_pad * n_pad) return;
    const int64_t g = (t >> 3) % g_pad;
    const int64_t n = (t / (g_pad * 8)) * 8 + (t & 7);
    const bool real = (g < G) && (n < N);
    if (scale_f16) {
        uint16_t v = real ? static_cast<const uint16_t*>(src)[g * N + n] : (uint16_t)0;
        const uint32_t mag = v & 0x7FFFu;
        const bool subnormal = (mag != 0u) && (mag < 0x0400u);
        const bool too_big = mag > 0x6FFFu;                  // |s| > 8188 or inf/nan
        if (subnormal || too_big) hdr[kHdrNoFold] = 1u;
        static_cast<uint16_t*>(dst)[t] = v;
    } else {
        float v = real ? static_cast<const float*>(src)[g * N + n] : 0.0f;
        static_cast<float*>(dst)[t] = v;
    }
}

hipError_t launch_pack(const uint8_t* codes, const void* scales, int scale_f16, int64_t N, int64_t K,
                       int64_t gs, const Layout& L, uint8_t* packed, hipStream_t s) {
    uint32_t* hdr = reinterpret_cast<uint32_t*>(packed);
    hipLaunchKernelGGL(clear_header_kernel, dim3(1), dim3(64), 0, s, hdr);
    const int64_t words = L.n_pad * (L.k_pad / 8);
    hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, codes, N,
                       K, L.n_pad, L.k_pad, reinterpret_cast<uint32_t*>(packed + L.nibble_offset), hdr);
    const int64_t nscale = L.g_pad * L.n_pad;
    hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((nscale + 255) / 256)), dim3(256), 0, s, scales,
                       scale_f16, N, K / gs, L.n_pad, L.g_pad, (void*)(packed + L.scale_offset), hdr);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void unpack_codes_kernel(const uint32_t* __restrict__ nib, int64_t N,
                                                           int64_t K, int64_t k_pad,
                                                           uint8_t* __restrict__ codes) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= N * K) return;
    const int64_t n = t / K;
    const int64_t k = t % K;
    const uint32_t word = nib[word_offset(k_pad, n, k >> 3) >> 2];
    codes[t] = (uint8_t)((word >> (4 * nib_pos((int)(k & 7)))) & 15u);
}

__global__ __launch_bounds__(256) void unpack_scales_kernel(const void* __restrict__ plane, int scale_f16,
                                                            int64_t N, int64_t G, int64_t g_pad,
                                                            void* __restrict__ dst) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= G * N) return;
    const int64_t g = t / N;
    const int64_t n = t % N;
    if (scale_f16)
        static_cast<uint16_t*>(dst)[t] = static_cast<const uint16_t*>(plane)[scale_index(g_pad, n, g)];
    else
        static_cast<float*>(dst)[t] = static_cast<const float*>(plane)[scale_index(g_pad, n, g)];
}

hipError_t launch_unpack(const WView& w, uint8_t* codes, void* scales, hipStream_t s) {
    const int64_t nk = w.N * w.K;
    hipLaunchKernelGGL(unpack_codes_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t*>(w.nib), w.N, w.K, w.k_pad, codes);
    const int64_t G = w.K / w.gs;
    const int64_t ng = G * w.N;
    hipLaunchKernelGGL(unpack_scales_kernel, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, s, w.scales,
                       w.scale_f16, w.N, G, w.g_pad, scales);
    return hipGetLastError();
}

}  // namespace q4gsw
