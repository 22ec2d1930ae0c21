// Generic q4gsw kernels: one lane per output element, fp32 VALU, any shape and any
// group size (including group sizes that are not multiples of 8).  They are the
// route of last resort; the fast routes cover the shapes the pages use.
#include "device.h"
#include "internal.h"

namespace q4gsw {

__device__ __forceinline__ int code_at(const uint8_t* nib, int64_t k_pad, int64_t n, int64_t k) {
    const uint32_t word = reinterpret_cast<const uint32_t*>(nib)[word_offset(k_pad, n, k >> 3) >> 2];
    return (int)((word >> (4 * nib_pos((int)(k & 7)))) & 15u);
}

// y[m, n] = sum_g scale[g, n] * sum_{k in g} x[m, k] * (code[n, k] - 8)
template <int XT>
__global__ __launch_bounds__(256) void generic_fwd_kernel(WView w, const void* __restrict__ x, int64_t M,
                                                          float* __restrict__ y) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= M * w.N) return;
    const int64_t m = t / w.N;
    const int64_t n = t % w.N;
    float acc = 0.0f;
    const int64_t G = w.K / w.gs;
    for (int64_t g = 0; g < G; ++g) {
        float part = 0.0f;
        for (int64_t k = g * w.gs; k < (g + 1) * w.gs; ++k) {
            const float a = load_elem<XT>(x, m * w.K + k);
            part = fmaf(a, (float)(code_at(w.nib, w.k_pad, n, k) - 8), part);
        }
        acc = fmaf(part, load_scale(w.scales, w.scale_f16, scale_index(w.g_pad, n, g)), acc);
    }
    y[t] = acc;
}

// d_x[m, k] = sum_n d_out[m, n] * scale[k / gs, n] * (code[n, k] - 8), summed in blocks of 64 n.
template <int GT>
__global__ __launch_bounds__(256) void generic_bwd_kernel(WView w, const void* __restrict__ d_out, int64_t M,
                                                          float* __restrict__ d_x) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= M * w.K) return;
    const int64_t m = t / w.K;
    const int64_t k = t % w.K;
    const int64_t g = k / w.gs;
    float acc = 0.0f;
    for (int64_t n0 = 0; n0 < w.N; n0 += 64) {
        float part = 0.0f;
        const int64_t n1 = n0 + 64 < w.N ? n0 + 64 : w.N;
        for (int64_t n = n0; n < n1; ++n) {
            const float d =
                load_elem<GT>(d_out, m * w.N + n) * load_scale(w.scales, w.scale_f16, scale_index(w.g_pad, n, g));
            part = fmaf(d, (float)(code_at(w.nib, w.k_pad, n, k) - 8), part);
        }
        acc += part;
    }
    d_x[t] = acc;
}

hipError_t launch_generic_fwd(const WView& w, const void* x, int x_dtype, int64_t M, float* y, hipStream_t s) {
    const int64_t total = M * w.N;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    switch (x_dtype) {
        case kF32: hipLaunchKernelGGL(generic_fwd_kernel<kF32>, grid, block, 0, s, w, x, M, y); break;
        case kF16: hipLaunchKernelGGL(generic_fwd_kernel<kF16>, grid, block, 0, s, w, x, M, y); break;
        default: hipLaunchKernelGGL(generic_fwd_kernel<kBF16>, grid, block, 0, s, w, x, M, y); break;
    }
    return hipGetLastError();
}

hipError_t launch_generic_bwd(const WView& w, const void* d_out, int g_dtype, int64_t M, float* d_x,
                              hipStream_t s) {
    const int64_t total = M * w.K;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    switch (g_dtype) {
        case kF32: hipLaunchKernelGGL(generic_bwd_kernel<kF32>, grid, block, 0, s, w, d_out, M, d_x); break;
        case kF16: hipLaunchKernelGGL(generic_bwd_kernel<kF16>, grid, block, 0, s, w, d_out, M, d_x); break;
        default: hipLaunchKernelGGL(generic_bwd_kernel<kBF16>, grid, block, 0, s, w, d_out, M, d_x); break;
    }
    return hipGetLastError();
}

}  // namespace q4gsw
