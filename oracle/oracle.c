/*
 * q4gsw oracle: a plain, slow, obviously correct CPU model of the 4-bit
 * group-symmetric weight-quantized linear layer, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library, and it includes no HIP header.
 *
 * What it computes (sources are the pages' own text):
 *
 *   dequant(W[n,k]) = (code[n,k] - 8) * scale[k / group_size, n]
 *       The dequantisation formula is given in the "Solution" part of the body of
 *       the pull request "[ExecuTorch][Vulkan] Add et_vk.linear_q4gsw_backward
 *       kernel (4-bit input-grad)"; its "Key changes" part gives the scale
 *       shape [num_groups, N].  The pages leave the scale's row index open; the
 *       plainest reading consistent with that shape (groups are contiguous runs
 *       of group_size along K) is k / group_size, integer division.
 *
 *   forward      y[m,n]  = sum_k x[m,k] * dequant(W[n,k])         (y = x . W^T)
 *       The forward is the linear_q4gsw op named on all three pages; the same
 *       pull request states its backward as the adjoint below, which fixes the
 *       forward as y = x . dequant(W)^T.
 *
 *   input grad   dx[m,k] = sum_n d_out[m,n] * dequant(W[n,k])     (contract N)
 *       Opening summary of the same Vulkan pull request body (the input
 *       gradient of the frozen 4-bit base, contracting over N).
 *
 *   embedding    out[t,k] = dequant(W[ids[t],k]): the embedding_q4gsw op named in a
 *       maintainer comment on the react-native-executorch issue "Upstream the Gemma 4
 *       Vulkan support we carry on our ExecuTorch fork" (its list of exporter changes),
 *       whose table may share the linear weight's layout (is_linear_weight, in the
 *       body of the WebGPU pull request that preserves the Q4 embedding's shader
 *       controls across resize).  Read plainly: row t of the output is row ids[t] of
 *       dequant(W).
 *       The pages say nothing of ids outside [0, N); here they give rows of zeros.
 *
 *   QKV          three forwards of one activation with three weights, three
 *       distinct outputs: body of "[ExecuTorch][WebGPU] Replace broad QKV
 *       fusion with BK64 kernel" (the QKV paragraph).  It is composed in the
 *       Python wrapper from three calls of oracle_linear_fwd.
 *
 *   dq8ca        the linear_dq8ca_q4gsw op named in the "Suggested split" of the
 *       react-native-executorch issue above: a linear whose activations are
 *       quantised to int8 on the fly.  The pages give only the op's name; the
 *       reading here ("dq8ca": dynamic int8, per channel of the activation, i.e. per
 *       row / token, asymmetric) is, for each row, with every step in fp32 as
 *       written and rint rounding half to even:
 *         lo = min(0, min_k x[k]),  hi = max(0, max_k x[k])    (zero stays exact)
 *         scale = (hi - lo) / 255, raised to the smallest normal fp32 if below it
 *         inv = 1 / scale
 *         zp = clamp(-128 - rint(lo * inv), -128, 127)
 *         q[k] = clamp(rint(x[k] * inv) + zp, -128, 127)
 *       and the row stands for scale * (q[k] - zp).  The linear is the forward
 *       above applied to those values, in fp64 (oracle_linear_dq8ca).
 *
 *   adapter step   The input-gradient pull request above says its op serves
 *       on-device adapter training around the frozen base; the same page lists, in
 *       its stack, an on-GPU AdamW optimizer step ("et_vk.adamw_step").  The pages
 *       give no adapter mathematics.  Reading: a rank-r low-rank adapter (LoRA, Hu
 *       et al., "LoRA: Low-Rank Adaptation of Large Language Models") beside the
 *       frozen q4gsw weight, A [r,K] and B [N,r] in fp32:
 *         t[m,j]   = sum_k x[m,k] A[j,k]
 *         y[m,n]   = sum_k x[m,k] dequant(W[n,k]) + alpha sum_j t[m,j] B[n,j]
 *       and, for an output gradient d_out, the gradients of <d_out, y>:
 *         u[m,j]   = sum_n d_out[m,n] B[n,j]
 *         dx[m,k]  = sum_n d_out[m,n] dequant(W[n,k]) + alpha sum_j u[m,j] A[j,k]
 *         dA[j,k]  = alpha sum_m u[m,j] x[m,k]
 *         dB[n,j]  = alpha sum_m d_out[m,n] t[m,j]
 *       The optimizer is AdamW as published (Loshchilov and Hutter, "Decoupled
 *       Weight Decay Regularization"), with bias-corrected moments and the weight
 *       decay applied to the parameter directly, for step s >= 1:
 *         p  <- p - lr wd p
 *         m  <- b1 m + (1 - b1) g,      v <- b2 v + (1 - b2) g^2
 *         p  <- p - lr (m / (1 - b1^s)) / (sqrt(v / (1 - b2^s)) + eps)
 *
 * Every input element is widened exactly to double: fp16 and bf16 are decoded
 * from their IEEE bit fields here.  Every product is exact in fp64 (at most
 * 24 + 3 + 24 significant bits); sums run with the contraction index
 * ascending, so the only rounding is the fp64 summation.  The normaliser
 * R = sum |activation| * |dequant(W)| over the same contraction is returned
 * beside every result; GPU results are judged against tol * R.
 *
 * Threads split the output elements only, so every sum keeps its order and the
 * results are bitwise identical for any thread count.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

enum {
    ORACLE_OK = 0,
    ORACLE_E_ARG = 1,        /* bad size, dtype or group size */
    ORACLE_E_CODE = 2,       /* a code outside 0..15 */
};

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exponent = (h >> 10) & 0x1f;
    int fraction = h & 0x3ff;
    double magnitude;
    if (exponent == 0) {
        magnitude = ldexp((double)fraction, -24);               /* subnormal or zero */
    } else if (exponent == 31) {
        magnitude = fraction ? NAN : INFINITY;
    } else {
        magnitude = ldexp((double)(fraction | 0x400), exponent - 25);
    }
    return sign ? -magnitude : magnitude;
}

/* bfloat16 is the upper half of an IEEE binary32: 1 sign, 8 exponent (bias 127), 7 fraction. */
double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int exponent = (b >> 7) & 0xff;
    int fraction = b & 0x7f;
    double magnitude;
    if (exponent == 0) {
        magnitude = ldexp((double)fraction, -133);
    } else if (exponent == 255) {
        magnitude = fraction ? NAN : INFINITY;
    } else {
        magnitude = ldexp((double)(fraction | 0x80), exponent - 134);
    }
    return sign ? -magnitude : magnitude;
}

/* IEEE binary32 read as bits: 1 sign, 8 exponent (bias 127), 23 fraction. */
double oracle_f32_to_f64(uint32_t u)
{
    int sign = (u >> 31) & 1;
    int exponent = (u >> 23) & 0xff;
    uint32_t fraction = u & 0x7fffffu;
    double magnitude;
    if (exponent == 0) {
        magnitude = ldexp((double)fraction, -149);
    } else if (exponent == 255) {
        magnitude = fraction ? NAN : INFINITY;
    } else {
        magnitude = ldexp((double)(fraction | 0x800000u), exponent - 150);
    }
    return sign ? -magnitude : magnitude;
}

static double element(const void *base, int dtype, int64_t index)
{
    if (dtype == ORACLE_F32) {
        uint32_t u;
        memcpy(&u, (const char *)base + 4 * index, 4);
        return oracle_f32_to_f64(u);
    }
    uint16_t h;
    memcpy(&h, (const char *)base + 2 * index, 2);
    return dtype == ORACLE_F16 ? oracle_f16_to_f64(h) : oracle_bf16_to_f64(h);
}

/* dequant(W[n,k]) = (code - 8) * scale[k / group_size, n]; scales are [K/group_size, N]. */
double oracle_dequant(const uint8_t *codes, const void *scales, int scale_dtype,
                      int64_t N, int64_t K, int64_t group_size, int64_t n, int64_t k)
{
    int code = codes[n * K + k];
    int64_t group = k / group_size;
    return (double)(code - 8) * element(scales, scale_dtype, group * N + n);
}

static int check_args(int act_dtype, int scale_dtype, int64_t M, int64_t N, int64_t K,
                      int64_t group_size, const uint8_t *codes)
{
    if (M < 0 || N < 0 || K < 0 || group_size <= 0 || K % group_size != 0)
        return ORACLE_E_ARG;
    if (act_dtype < ORACLE_F32 || act_dtype > ORACLE_BF16)
        return ORACLE_E_ARG;
    if (scale_dtype != ORACLE_F32 && scale_dtype != ORACLE_F16)
        return ORACLE_E_ARG;
    for (int64_t i = 0; i < N * K; ++i)
        if (codes[i] > 15)
            return ORACLE_E_CODE;
    return ORACLE_OK;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* y[m,n] = sum_k x[m,k] * dequant(W[n,k]); r[m,n] = sum_k |x[m,k]| * |dequant(W[n,k])|.
 * x is [M,K] row-major in act_dtype; codes [N,K]; y and r (r may be NULL) are [M,N]. */
int oracle_linear_fwd(const void *x, int act_dtype, int64_t M,
                      const uint8_t *codes, const void *scales, int scale_dtype,
                      int64_t N, int64_t K, int64_t group_size,
                      double *y, double *r, int nthreads)
{
    int status = check_args(act_dtype, scale_dtype, M, N, K, group_size, codes);
    if (status != ORACLE_OK)
        return status;
    set_threads(nthreads);
    int64_t outputs = M * N;
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < outputs; ++o) {
        int64_t m = o / N, n = o % N;
        double sum = 0.0, norm = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = element(x, act_dtype, m * K + k);
            double w = oracle_dequant(codes, scales, scale_dtype, N, K, group_size, n, k);
            sum += a * w;
            norm += fabs(a) * fabs(w);
        }
        y[o] = sum;
        if (r)
            r[o] = norm;
    }
    return ORACLE_OK;
}

/* dx[m,k] = sum_n d_out[m,n] * dequant(W[n,k]); r[m,k] = sum_n |d_out[m,n]| * |dequant(W[n,k])|.
 * d_out is [M,N] row-major in act_dtype; codes [N,K]; dx and r (r may be NULL) are [M,K]. */
int oracle_linear_bwd_input(const void *d_out, int act_dtype, int64_t M,
                            const uint8_t *codes, const void *scales, int scale_dtype,
                            int64_t N, int64_t K, int64_t group_size,
                            double *dx, double *r, int nthreads)
{
    int status = check_args(act_dtype, scale_dtype, M, N, K, group_size, codes);
    if (status != ORACLE_OK)
        return status;
    set_threads(nthreads);
    int64_t outputs = M * K;
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < outputs; ++o) {
        int64_t m = o / K, k = o % K;
        double sum = 0.0, norm = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double g = element(d_out, act_dtype, m * N + n);
            double w = oracle_dequant(codes, scales, scale_dtype, N, K, group_size, n, k);
            sum += g * w;
            norm += fabs(g) * fabs(w);
        }
        dx[o] = sum;
        if (r)
            r[o] = norm;
    }
    return ORACLE_OK;
}

/* out[t,k] = dequant(W[ids[t],k]) for ids[t] in [0, N), else 0; ids has T entries, out is [T,K]. */
int oracle_embedding(const int64_t *ids, int64_t T, const uint8_t *codes, const void *scales,
                     int scale_dtype, int64_t N, int64_t K, int64_t group_size, double *out)
{
    int status = check_args(ORACLE_F32, scale_dtype, T, N, K, group_size, codes);
    if (status != ORACLE_OK)
        return status;
    for (int64_t t = 0; t < T; ++t) {
        int64_t n = ids[t];
        for (int64_t k = 0; k < K; ++k)
            out[t * K + k] = (n >= 0 && n < N)
                                 ? oracle_dequant(codes, scales, scale_dtype, N, K, group_size, n, k)
                                 : 0.0;
    }
    return ORACLE_OK;
}

/* The number of OpenMP threads a parallel region would use after set_threads(nthreads). */
/* Per-row int8 quantisation of the activation (the dq8ca reading in the header).  The
 * arithmetic is fp32 on purpose: it decides integers, and the GPU takes the same decisions in
 * the same precision.  Outputs: q [M, K] int8, scale [M] fp32, zp [M] int32. */
int oracle_dq8ca_quantize(const void *x, int act_dtype, int64_t M, int64_t K,
                          int8_t *q, float *scale, int32_t *zp, int nthreads)
{
    if (M < 1 || K < 1 || act_dtype < ORACLE_F32 || act_dtype > ORACLE_BF16) return ORACLE_E_ARG;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float lo = 0.0f, hi = 0.0f;
        for (int64_t i = 0; i < K; ++i) {
            const float v = (float)element(x, act_dtype, m * K + i);    /* exact: an fp32/fp16/bf16 value */
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        float s = (hi - lo) / 255.0f;
        if (s < FLT_MIN) s = FLT_MIN;
        const float inv = 1.0f / s;
        int z = -128 - (int)rintf(lo * inv);
        if (z < -128) z = -128;
        if (z > 127) z = 127;
        for (int64_t i = 0; i < K; ++i) {
            const float v = (float)element(x, act_dtype, m * K + i);
            int t = (int)rintf(v * inv) + z;
            if (t < -128) t = -128;
            if (t > 127) t = 127;
            q[m * K + i] = (int8_t)t;
        }
        scale[m] = s;
        zp[m] = z;
    }
    return ORACLE_OK;
}

/* The linear on the quantised rows: y[m,n] = sum_k scale[m] * (q[m,k] - zp[m]) * dequant(W[n,k]),
 * in fp64 with k ascending, and its normaliser R = sum |scale[m] * (q - zp)| * |dequant(W[n,k])|. */
int oracle_linear_dq8ca(const int8_t *q, const float *scale, const int32_t *zp, int64_t M,
                        const uint8_t *codes, const void *scales, int scale_dtype,
                        int64_t N, int64_t K, int64_t group_size, double *y, double *norm, int nthreads)
{
    int st = check_args(ORACLE_F32, scale_dtype, M, N, K, group_size, codes);
    if (st != ORACLE_OK) return st;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < M * N; ++o) {
        const int64_t m = o / N;
        const int64_t n = o - m * N;
        double acc = 0.0, nrm = 0.0;
        const double sm = (double)scale[m];
        for (int64_t k = 0; k != K; ++k) {
            double a = sm * (double)((int)q[m * K + k] - (int)zp[m]);
            double w = oracle_dequant(codes, scales, scale_dtype, N, K, group_size, n, k);
            acc += a * w;
            nrm += fabs(a) * fabs(w);
        }
        y[o] = acc;
        norm[o] = nrm;
    }
    return ORACLE_OK;
}

/* codes == NULL in the adapter calls below: the frozen-weight term is left out, so y (or dx)
 * and its normaliser hold the adapter term alone (for checking the factors at sizes where the
 * dense term would take too long). */
static int adapter_only_args(int act_dtype, int64_t M, int64_t N, int64_t K, double *out, double *r)
{
    if (M < 0 || N < 0 || K < 0 || act_dtype < ORACLE_F32 || act_dtype > ORACLE_BF16)
        return ORACLE_E_ARG;
    for (int64_t i = 0; i < M * N; ++i) {
        out[i] = 0.0;
        if (r)
            r[i] = 0.0;
    }
    return ORACLE_OK;
}

/* The adapter forward (see the header): y and its normaliser r are [M,N], t = x A^T is [M,r].
 * r[m,n] = sum_k |x||dequant(W)| + |alpha| sum_j (sum_k |x[m,k]| |A[j,k]|) |B[n,j]|. */
int oracle_lora_fwd(const void *x, int act_dtype, int64_t M,
                    const uint8_t *codes, const void *scales, int scale_dtype,
                    int64_t N, int64_t K, int64_t group_size,
                    const float *A, const float *B, int64_t rank, double alpha,
                    double *y, double *t, double *r, int nthreads)
{
    int status = codes ? oracle_linear_fwd(x, act_dtype, M, codes, scales, scale_dtype, N, K, group_size, y, r,
                                           nthreads)
                       : adapter_only_args(act_dtype, M, N, K, y, r);
    if (status != ORACLE_OK)
        return status;
    if (rank < 0)
        return ORACLE_E_ARG;
    /* t = x A^T and its absolute counterpart, row by row */
    for (int64_t row = 0; row < M; ++row) {
        for (int64_t j = 0; j < rank; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t c = 0; c < K; ++c) {
                double a = element(x, act_dtype, row * K + c);
                acc += a * (double)A[j * K + c];
                mag += fabs(a) * fabs((double)A[j * K + c]);
            }
            t[row * rank + j] = acc;
            for (int64_t col = 0; col < N; ++col) {
                y[row * N + col] += alpha * acc * (double)B[col * rank + j];
                if (r)
                    r[row * N + col] += fabs(alpha) * mag * fabs((double)B[col * rank + j]);
            }
        }
    }
    return ORACLE_OK;
}

/* The adapter backward (see the header).  d_out is [M,N] in act_dtype, x [M,K] in act_dtype.
 * dx and rdx are [M,K]; dA and rdA [rank,K]; dB and rdB [N,rank].  Each r* is the sum of the
 * absolute values of the products its output sums (the base part of rdx as for the input
 * gradient). */
int oracle_lora_bwd(const void *x, const void *d_out, int act_dtype, int64_t M,
                    const uint8_t *codes, const void *scales, int scale_dtype,
                    int64_t N, int64_t K, int64_t group_size,
                    const float *A, const float *B, int64_t rank, double alpha,
                    double *dx, double *dA, double *dB, double *rdx, double *rdA, double *rdB, int nthreads)
{
    int status = codes ? oracle_linear_bwd_input(d_out, act_dtype, M, codes, scales, scale_dtype, N, K, group_size,
                                                 dx, rdx, nthreads)
                       : adapter_only_args(act_dtype, M, K, N, dx, rdx);
    if (status != ORACLE_OK)
        return status;
    if (rank < 0)
        return ORACLE_E_ARG;
    for (int64_t i = 0; i < rank * K; ++i) {
        dA[i] = 0.0;
        rdA[i] = 0.0;
    }
    for (int64_t i = 0; i < N * rank; ++i) {
        dB[i] = 0.0;
        rdB[i] = 0.0;
    }
    for (int64_t row = 0; row < M; ++row) {
        for (int64_t j = 0; j < rank; ++j) {
            /* u[row,j] = sum_n d_out[row,n] B[n,j]; tx[row,j] = sum_k x[row,k] A[j,k] */
            double u = 0.0, umag = 0.0, tx = 0.0, tmag = 0.0;
            for (int64_t col = 0; col < N; ++col) {
                double g = element(d_out, act_dtype, row * N + col);
                u += g * (double)B[col * rank + j];
                umag += fabs(g) * fabs((double)B[col * rank + j]);
            }
            for (int64_t c = 0; c < K; ++c) {
                double a = element(x, act_dtype, row * K + c);
                tx += a * (double)A[j * K + c];
                tmag += fabs(a) * fabs((double)A[j * K + c]);
            }
            for (int64_t c = 0; c < K; ++c) {
                double a = element(x, act_dtype, row * K + c);
                dx[row * K + c] += alpha * u * (double)A[j * K + c];
                rdx[row * K + c] += fabs(alpha) * umag * fabs((double)A[j * K + c]);
                dA[j * K + c] += alpha * u * a;
                rdA[j * K + c] += fabs(alpha) * umag * fabs(a);
            }
            for (int64_t col = 0; col < N; ++col) {
                double g = element(d_out, act_dtype, row * N + col);
                dB[col * rank + j] += alpha * g * tx;
                rdB[col * rank + j] += fabs(alpha) * fabs(g) * tmag;
            }
        }
    }
    return ORACLE_OK;
}

/* One AdamW step (see the header) on n fp32 parameters, in fp64: p_out, m_out, v_out. */
int oracle_adamw(const float *p, const float *g, const float *m, const float *v, int64_t n,
                 double lr, double beta1, double beta2, double eps, double weight_decay, int64_t step,
                 double *p_out, double *m_out, double *v_out)
{
    if (n < 0 || step < 1)
        return ORACLE_E_ARG;
    const double bias1 = 1.0 - pow(beta1, (double)step);
    const double bias2 = 1.0 - pow(beta2, (double)step);
    for (int64_t i = 0; i < n; ++i) {
        double param = (double)p[i];
        const double grad = (double)g[i];
        param -= lr * weight_decay * param;
        const double m1 = beta1 * (double)m[i] + (1.0 - beta1) * grad;
        const double v1 = beta2 * (double)v[i] + (1.0 - beta2) * grad * grad;
        param -= lr * (m1 / bias1) / (sqrt(v1 / bias2) + eps);
        p_out[i] = param;
        m_out[i] = m1;
        v_out[i] = v1;
    }
    return ORACLE_OK;
}

int oracle_threads(int nthreads)
{
    set_threads(nthreads);
#ifdef _OPENMP
    int used = 1;
#pragma omp parallel
    {
#pragma omp single
        used = omp_get_num_threads();
    }
    return used;
#else
    return 1;
#endif
}
