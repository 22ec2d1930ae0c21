/*
 * q4gsw: the 4-bit group-symmetric weight-quantized linear layer on AMD MI355X (gfx950).
 *
 * The operation (sources are the pages this library is built from):
 *
 *   dequant(W[n,k]) = (code[n,k] - 8) * scale[k / group_size, n]
 *       codes are 4-bit (0..15); scales are [num_groups, N] with
 *       num_groups = K / group_size.  Formula: "Solution" part of the body of
 *       "[ExecuTorch][Vulkan] Add et_vk.linear_q4gsw_backward kernel (4-bit
 *       input-grad)"; scale shape: the "Key changes" part of that body.  The
 *       row index k / group_size is the reading of that shape in which groups
 *       are contiguous runs of group_size along K.
 *
 *   forward          y[M,N]   = x[M,K] . dequant(W)[N,K]^T
 *   input gradient   d_x[M,K] = d_out[M,N] . dequant(W)[N,K], contracting over N
 *       (opening summary of the same Vulkan body: the input gradient of a frozen
 *       4-bit base, for adapter training; there is no weight gradient).
 *   fused QKV        q, k, v = x . dequant(Wq)^T, x . dequant(Wk)^T, x . dequant(Wv)^T
 *       (body of "[ExecuTorch][WebGPU] Replace broad QKV fusion with BK64 kernel":
 *       one activation, three weights packed once, three distinct outputs).
 *
 * Conventions for every call:
 *   - Every tensor is dense and row-major.  Every data pointer is a device
 *     pointer owned by the caller; the library never allocates device memory.
 *   - Arguments are validated on the host before any HIP call.  A call that
 *     fails validation returns a status other than Q4GSW_OK, launches nothing
 *     and leaves every output untouched.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Compute calls are
 *     asynchronous on it; only q4gsw_pack and q4gsw_unpack synchronize it.
 *   - Outputs are fp32.  Activations may be fp32, fp16 or bf16; scales fp16 or
 *     fp32.  Accumulation is fp32.
 *   - No C++ exception crosses this interface.  Calls are independent: route and
 *     plan choices are per call (q4gsw_options), never process-wide.  The state
 *     the library keeps: a cache of resident blocks per CU for each kernel
 *     instance (filled on first use from the HIP occupancy query, then read-only;
 *     a race between threads only repeats the same query), and, for
 *     q4gsw_linear_fwd_noalloc, one scratch array per device with its address
 *     (shared by every call of that entry point on the device; see there).
 */
#ifndef Q4GSW_H
#define Q4GSW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4GSW_MAGIC 0x57534734u          /* "4GSW" */
#define Q4GSW_LAYOUT_VERSION 2u

typedef enum q4gsw_status {
    Q4GSW_OK = 0,
    Q4GSW_E_NULL = 1,         /* a required pointer is NULL */
    Q4GSW_E_SHAPE = 2,        /* a size is out of range (M, N or K < 1, or too large) */
    Q4GSW_E_DTYPE = 3,        /* an unsupported dtype code */
    Q4GSW_E_GROUP = 4,        /* group_size < 1 or K % group_size != 0 */
    Q4GSW_E_ALIAS = 5,        /* an output overlaps another output, an input or the workspace */
    Q4GSW_E_CODE_RANGE = 6,   /* q4gsw_pack saw a code above 15 */
    Q4GSW_E_WORKSPACE = 7,    /* workspace missing, smaller than q4gsw_*_workspace_bytes or not 256-byte aligned */
    Q4GSW_E_DESC = 8,         /* descriptor magic/version/fields invalid, or QKV weights disagree */
    Q4GSW_E_HIP = 9,          /* a HIP runtime call or kernel launch failed */
    Q4GSW_E_BUFFER = 10,      /* packed buffer smaller than q4gsw_packed_bytes */
    Q4GSW_E_ROUTE = 11,       /* the route requested in q4gsw_options cannot serve this call */
    Q4GSW_E_SCRATCH = 12      /* q4gsw_linear_fwd_noalloc: the call needs more than Q4GSW_SCRATCH_BYTES */
} q4gsw_status;

typedef enum q4gsw_dtype {
    Q4GSW_F32 = 0,
    Q4GSW_F16 = 1,
    Q4GSW_BF16 = 2
} q4gsw_dtype;

typedef enum q4gsw_op {
    Q4GSW_OP_FWD = 0,
    Q4GSW_OP_BWD_INPUT = 1,
    Q4GSW_OP_QKV = 2,
    Q4GSW_OP_DQ8CA = 3           /* q4gsw_linear_dq8ca */
} q4gsw_op;

/* Kernel routes, reported by q4gsw_route (route attestation). */
typedef enum q4gsw_route_id {
    Q4GSW_ROUTE_NONE = 0,          /* the call would fail validation */
    Q4GSW_ROUTE_GENERIC = 1,       /* VALU, one lane per output, any shape and group size */
    Q4GSW_ROUTE_GEMV = 2,          /* forward, M <= 8: bandwidth-bound streaming GEMV */
    Q4GSW_ROUTE_GEMM_FOLD = 3,     /* forward, fp16 x: MFMA f16, scale folded into the fp16 weight */
    Q4GSW_ROUTE_GEMM_GROUP = 4,    /* forward, fp16/bf16 x: MFMA on exact codes, fp32 scale per group */
    Q4GSW_ROUTE_GEMM_SPLIT = 5,    /* forward, fp32 x: x split into bf16 hi+lo, two MFMA passes */
    Q4GSW_ROUTE_BWD_GEMV = 6,      /* input gradient, M <= 8: streaming transposed GEMV */
    Q4GSW_ROUTE_BWD_FOLD = 7,      /* input gradient, fp16 d_out: MFMA f16 on folded fp16 weight */
    Q4GSW_ROUTE_BWD_SPLIT = 8,     /* input gradient: d_out*scale split into bf16 hi+lo, two MFMA passes */
    Q4GSW_ROUTE_QKV_FUSED = 9,     /* fused QKV: one launch over the three weights */
    Q4GSW_ROUTE_BWD_BSPLIT = 10,   /* input gradient, fp16 scales, gs % 64 == 0 or 32: d_out in bf16 hi+lo
                                      planes, (code - 8) * scale split exactly into bf16 hi+lo, 2 or 4 passes */
    Q4GSW_ROUTE_DQ8CA = 11         /* q4gsw_linear_dq8ca: per-row int8 activations, int8 MFMA */
} q4gsw_route_id;

/*
 * Per-call route and plan choice, for tests and benchmarks that compare routes and
 * plans (the caller picks, q4gsw_plan reports).  All zero, or a NULL pointer,
 * leaves every choice to the library; the plain calls take none.
 *   route      Q4GSW_ROUTE_NONE: automatic.  Otherwise the route family to take:
 *              GENERIC; a small-M route (GEMV, BWD_GEMV); or an MFMA route (any of
 *              GEMM_FOLD, GEMM_GROUP, GEMM_SPLIT, BWD_FOLD, BWD_SPLIT, BWD_BSPLIT, QKV_FUSED:
 *              the library picks the precision route inside the family).  A call
 *              the family cannot serve returns Q4GSW_E_ROUTE; a value outside the
 *              enum returns Q4GSW_E_ROUTE too.
 *   tile_rows  forward / QKV MFMA block rows: 0 (per shape), 64 or 128 (fp32 activations always
 *              take 64: their mode has no 128-row tile)
 *              (Q4GSW_E_SHAPE otherwise).
 *   splits     contraction splits of the 32x32 MFMA GEMMs (forward, QKV and the
 *              input-gradient routes BWD_FOLD, BWD_SPLIT and BWD_BSPLIT): 0 (per shape) or
 *              1..64 (Q4GSW_E_SHAPE otherwise), clamped to the 64-wide chunks and
 *              rounded to a count with no empty split.
 * A workspace is sized for the options it is used with (q4gsw_*_workspace_bytes_ex).
 */
typedef struct q4gsw_options {
    int32_t route;
    int32_t tile_rows;
    int32_t splits;
} q4gsw_options;

/*
 * Packed weight descriptor, filled by q4gsw_pack.  Plain data: copy it freely.
 * `data` points into the caller's packed buffer; the descriptor does not own it.
 * A descriptor is immutable after packing and serves every M (one prepack,
 * reused by forward, input gradient and QKV).
 */
typedef struct q4gsw_weight {
    uint32_t magic;           /* Q4GSW_MAGIC */
    uint32_t version;         /* Q4GSW_LAYOUT_VERSION */
    int64_t N;                /* output features (rows of W) */
    int64_t K;                /* input features (columns of W) */
    int64_t group_size;       /* K-run sharing one scale */
    int64_t n_pad;            /* N rounded up to the packing tile */
    int64_t k_pad;            /* K rounded up to the packing tile */
    int64_t g_pad;            /* scale groups stored: ceil(k_pad / group_size) */
    int32_t scale_dtype;      /* Q4GSW_F16 or Q4GSW_F32 */
    uint32_t flags;           /* Q4GSW_FLAG_* set by q4gsw_pack */
    void *data;               /* device pointer to the packed buffer */
    uint64_t bytes;           /* bytes of the packed buffer in use */
    uint64_t nibble_offset;   /* byte offset of the 4-bit code plane */
    uint64_t scale_offset;    /* byte offset of the scale plane (g_pad * n_pad scales) */
} q4gsw_weight;

/* Set by q4gsw_pack when every fp16 scale s is 0 or 2^-14 <= |s| <= 8188, so that
 * (code - 8) * s is a finite normal fp16 (rounding error at most 2^-11 relative). */
#define Q4GSW_FLAG_FOLD_F16 1u

/* Bytes of the packed buffer for an [N, K] weight.  Pure host function.
 * Returns E_SHAPE, E_GROUP or E_DTYPE on bad arguments, E_NULL if bytes is NULL. */
q4gsw_status q4gsw_packed_bytes(int64_t N, int64_t K, int64_t group_size, int32_t scale_dtype,
                                uint64_t *bytes);

/*
 * One-time repack of the codes and scales into the gfx950 layout (the prepack
 * that forward, input gradient and QKV all reuse).  The Vulkan q4gsw-backward
 * pull request ("Key changes") reuses the forward's prepacked weight and scales
 * in the backward with no re-pack, and the WebGPU BK64 QKV pull request body
 * packs the constant weights and scales once; this call is that one packing step,
 * into a layout of this library's own.
 *   codes   device, uint8 [N, K], one code (0..15) per byte
 *   scales  device, [K / group_size, N] in scale_dtype (Q4GSW_F16 or Q4GSW_F32)
 *   packed  device, at least q4gsw_packed_bytes(...) bytes; overwritten
 *   out     host descriptor, filled on success
 * Synchronizes `stream` to read back the code-range check.  Returns
 * E_CODE_RANGE if any code exceeds 15 (the packed buffer is then undefined and
 * `out` is left untouched).
 */
q4gsw_status q4gsw_pack(const uint8_t *codes, const void *scales, int32_t scale_dtype,
                        int64_t N, int64_t K, int64_t group_size,
                        void *packed, uint64_t packed_bytes, void *stream, q4gsw_weight *out);

/* The exact inverse of q4gsw_pack: writes codes [N, K] uint8 and scales
 * [K / group_size, N] in the weight's scale dtype.  Synchronizes `stream`.
 * It makes the packing of the passages cited at q4gsw_pack checkable: the
 * packed buffer holds exactly the caller's codes and scales, bit for bit.
 * E_DESC for a bad descriptor, E_NULL for a null output, E_ALIAS when the
 * outputs overlap each other or the packed buffer. */
q4gsw_status q4gsw_unpack(const q4gsw_weight *w, uint8_t *codes, void *scales, void *stream);

/* Device workspace (bytes) the call needs; 0 when its route needs none.  Pure host.  A workspace
 * passed to a call that needs one must start on a 256-byte boundary (E_WORKSPACE otherwise); its
 * contents need no initialisation and are scratch after the call. */
q4gsw_status q4gsw_workspace_bytes(int32_t op, const q4gsw_weight *w, int64_t M, int32_t act_dtype,
                                   uint64_t *bytes);
q4gsw_status q4gsw_qkv_workspace_bytes(const q4gsw_weight *wq, const q4gsw_weight *wk,
                                       const q4gsw_weight *wv, int64_t M, int32_t x_dtype,
                                       uint64_t *bytes);
/* The same sizes for a call made with `opts` (NULL: as above). */
q4gsw_status q4gsw_workspace_bytes_ex(int32_t op, const q4gsw_weight *w, int64_t M, int32_t act_dtype,
                                      const q4gsw_options *opts, uint64_t *bytes);
q4gsw_status q4gsw_qkv_workspace_bytes_ex(const q4gsw_weight *wq, const q4gsw_weight *wk,
                                          const q4gsw_weight *wv, int64_t M, int32_t x_dtype,
                                          const q4gsw_options *opts, uint64_t *bytes);

/*
 * Forward: y[M, N] (fp32) = x[M, K] . dequant(W)^T.
 *   x   device [M, K] in x_dtype (Q4GSW_F32, Q4GSW_F16, Q4GSW_BF16)
 *   y   device fp32 [M, N]; must not overlap x, the packed weight or the workspace
 *   ws  device workspace of ws_bytes >= q4gsw_workspace_bytes(Q4GSW_OP_FWD, ...)
 *       (may be NULL when that is 0)
 */
q4gsw_status q4gsw_linear_fwd(const q4gsw_weight *w, const void *x, int32_t x_dtype, int64_t M,
                              float *y, void *ws, uint64_t ws_bytes, void *stream);
/* q4gsw_linear_fwd with per-call options (NULL: the same call). */
q4gsw_status q4gsw_linear_fwd_ex(const q4gsw_weight *w, const void *x, int32_t x_dtype, int64_t M,
                                 float *y, void *ws, uint64_t ws_bytes, const q4gsw_options *opts,
                                 void *stream);

/*
 * Forward that allocates nothing and takes no workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same routes, kernels and results as q4gsw_linear_fwd with no options (bit for
 * bit).  The split partials that q4gsw_linear_fwd keeps in the caller's workspace go to a
 * scratch buffer of Q4GSW_SCRATCH_BYTES that the library holds on each device from module load
 * until the process ends.  A call whose workspace (q4gsw_workspace_bytes) would exceed it
 * returns Q4GSW_E_SCRATCH and launches nothing.  Every call on one device shares that device's
 * buffer and nothing in it needs to start at zero: calls that overlap on one device (other
 * streams or host threads) race on it, so the caller must order them.  Other errors as
 * q4gsw_linear_fwd (E_HIP also if the scratch address cannot be obtained).
 */
#define Q4GSW_SCRATCH_BYTES (32u << 20)
q4gsw_status q4gsw_linear_fwd_noalloc(const q4gsw_weight *w, const void *x, int32_t x_dtype, int64_t M,
                                      float *y, void *stream);

/*
 * Input gradient: d_x[M, K] (fp32) = d_out[M, N] . dequant(W), contracting over N.
 * Reads the same packed buffer as the forward (no re-pack).
 *   d_out  device [M, N] in g_dtype;  d_x device fp32 [M, K]
 */
q4gsw_status q4gsw_linear_bwd_input(const q4gsw_weight *w, const void *d_out, int32_t g_dtype,
                                    int64_t M, float *d_x, void *ws, uint64_t ws_bytes,
                                    void *stream);
/* q4gsw_linear_bwd_input with per-call options (NULL: the same call). */
q4gsw_status q4gsw_linear_bwd_input_ex(const q4gsw_weight *w, const void *d_out, int32_t g_dtype,
                                       int64_t M, float *d_x, void *ws, uint64_t ws_bytes,
                                       const q4gsw_options *opts, void *stream);

/*
 * Fused QKV: q = x . dequant(Wq)^T, k = x . dequant(Wk)^T, v = x . dequant(Wv)^T.
 * The three weights must share K, group_size and scale dtype (E_DESC otherwise);
 * their N may differ.  q [M, Nq], k [M, Nk], v [M, Nv] are fp32 and must not
 * overlap each other, x, the packed weights or the workspace (E_ALIAS).
 * Shapes outside the fused kernel's predicate run as three forwards with the
 * same result contract.
 */
q4gsw_status q4gsw_qkv_fused(const q4gsw_weight *wq, const q4gsw_weight *wk, const q4gsw_weight *wv,
                             const void *x, int32_t x_dtype, int64_t M,
                             float *q, float *k, float *v, void *ws, uint64_t ws_bytes,
                             void *stream);
/* q4gsw_qkv_fused with per-call options (NULL: the same call). */
q4gsw_status q4gsw_qkv_fused_ex(const q4gsw_weight *wq, const q4gsw_weight *wk, const q4gsw_weight *wv,
                                const void *x, int32_t x_dtype, int64_t M,
                                float *q, float *k, float *v, void *ws, uint64_t ws_bytes,
                                const q4gsw_options *opts, void *stream);

/*
 * Per-row int8 quantisation of activations, the activation side of linear_dq8ca_q4gsw (the
 * "Suggested split" of the react-native-executorch issue "Upstream the Gemma 4 Vulkan support we
 * carry on our ExecuTorch fork" names the op and nothing more).  Reading: per row (token),
 * asymmetric, zero exact, every step in fp32 as written, rint rounding half to even:
 *   lo = min(0, min x), hi = max(0, max x), scale = (hi - lo) / 255 (at least the smallest
 *   normal fp32), inv = 1 / scale, zero_point = clamp(-128 - rint(lo * inv), -128, 127),
 *   q = clamp(rint(x * inv) + zero_point, -128, 127); the row stands for scale * (q - zero_point).
 *   x           device [M, K] in x_dtype (Q4GSW_F32, Q4GSW_F16, Q4GSW_BF16)
 *   q           device int8 [M, K];  scale device fp32 [M];  zero_point device int32 [M]
 * E_NULL, E_SHAPE (M or K < 1 or too large), E_DTYPE, E_ALIAS (outputs overlap each other or x).
 */
q4gsw_status q4gsw_dq8ca_quantize(const void *x, int32_t x_dtype, int64_t M, int64_t K, int8_t *q,
                                  float *scale, int32_t *zero_point, void *stream);

/*
 * linear_dq8ca_q4gsw: y[M, N] (fp32) = (scale * (q - zero_point)) . dequant(W)^T, the forward on
 * the rows q4gsw_dq8ca_quantize makes of x, quantised on the fly (int8 MFMA; the zero point is
 * applied exactly in int32, the scales in fp32).  Same packed weight as the forward.
 *   x   device [M, K] in x_dtype;  y device fp32 [M, N]
 *   ws  device workspace of ws_bytes >= q4gsw_workspace_bytes(Q4GSW_OP_DQ8CA, ...) (never 0:
 *       it holds the quantised rows); contents need no initialisation
 * E_GROUP when group_size is neither 32 nor a multiple of 64; other errors as q4gsw_linear_fwd.
 */
q4gsw_status q4gsw_linear_dq8ca(const q4gsw_weight *w, const void *x, int32_t x_dtype, int64_t M, float *y,
                                void *ws, uint64_t ws_bytes, void *stream);
/* q4gsw_linear_dq8ca with per-call options (only `splits` applies; NULL: the same call). */
q4gsw_status q4gsw_linear_dq8ca_ex(const q4gsw_weight *w, const void *x, int32_t x_dtype, int64_t M, float *y,
                                   void *ws, uint64_t ws_bytes, const q4gsw_options *opts, void *stream);

/*
 * The adapter step around the frozen base.  The Vulkan pull request "[ExecuTorch][Vulkan] Add
 * et_vk.linear_q4gsw_backward kernel (4-bit input-grad)" says (opening summary) that the input
 * gradient serves on-device adapter training around the frozen 4-bit base, and its stack lists an
 * on-GPU AdamW optimizer step (et_vk.adamw_step); the pages give no adapter mathematics.
 * Reading: a rank-r low-rank adapter beside the packed weight, factors A [r, K] and B [N, r] in
 * fp32 row-major, scaled by alpha:
 *   t = x A^T [M, r],    y = x . dequant(W)^T + alpha t B^T
 * and, for the loss <d_out, y>,
 *   u = d_out B,  d_x = d_out . dequant(W) + alpha u A,  d_A = alpha u^T x,  d_B = alpha d_out^T t.
 * Both calls run the library's forward / input gradient for the W term (its routes and precision)
 * and fp32 kernels for the low-rank terms, every sum in a fixed order (results do not depend on
 * the launch).  rank: 1..64.
 *
 * q4gsw_adapter_workspace_bytes: workspace of q4gsw_adapter_fwd (op Q4GSW_OP_FWD) or
 * q4gsw_adapter_bwd (op Q4GSW_OP_BWD_INPUT) for M rows of act_dtype at this rank.
 * E_NULL, E_DESC, E_SHAPE (M, rank or op out of range), E_DTYPE.
 */
q4gsw_status q4gsw_adapter_workspace_bytes(int32_t op, const q4gsw_weight *w, int64_t M, int32_t act_dtype,
                                           int32_t rank, uint64_t *bytes);
/*
 *   x  device [M, K] in x_dtype;  A device fp32 [rank, K];  B device fp32 [N, rank]
 *   y  device fp32 [M, N] (written);  t device fp32 [M, rank] (written: x A^T, kept for the backward)
 *   ws device workspace of ws_bytes (256-byte aligned) >= q4gsw_adapter_workspace_bytes(Q4GSW_OP_FWD)
 * E_NULL, E_SHAPE (rank, M, non-finite alpha), E_DTYPE, E_GROUP, E_WORKSPACE, E_ALIAS (an output
 * overlaps an input, the other output or the workspace), E_HIP.
 */
q4gsw_status q4gsw_adapter_fwd(const q4gsw_weight *w, const void *x, int32_t x_dtype, int64_t M, const float *A,
                               const float *B, int32_t rank, float alpha, float *y, float *t, void *ws,
                               uint64_t ws_bytes, void *stream);
/*
 *   x, d_out  device [M, K] and [M, N] in dtype (one dtype for both);  A, B, t as above (t from the
 *             forward of the same x)
 *   d_x device fp32 [M, K];  d_A device fp32 [rank, K];  d_B device fp32 [N, rank] (all written)
 *   ws  device workspace (256-byte aligned) >= q4gsw_adapter_workspace_bytes(Q4GSW_OP_BWD_INPUT):
 *       the input gradient's, then u [M, rank]
 * Errors as q4gsw_adapter_fwd; outputs may overlap neither each other, any input nor ws.
 */
q4gsw_status q4gsw_adapter_bwd(const q4gsw_weight *w, const void *x, const void *d_out, int32_t dtype, int64_t M,
                               const float *A, const float *B, int32_t rank, float alpha, const float *t, float *d_x,
                               float *d_A, float *d_B, void *ws, uint64_t ws_bytes, void *stream);

/*
 * One AdamW step (Loshchilov and Hutter, "Decoupled Weight Decay Regularization": decoupled decay,
 * bias-corrected moments) on n fp32 values in place, for step >= 1:
 *   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
 *   p <- p - lr / (1 - b1^step) * m / (sqrt(v) / sqrt(1 - b2^step) + eps)
 * param, exp_avg (m), exp_avg_sq (v): device fp32 [n], updated;  grad: device fp32 [n].
 * E_NULL, E_SHAPE (n < 0, step < 1, lr or wd negative or not finite, beta outside [0, 1), eps not
 * positive and finite), E_ALIAS (any two buffers overlap), E_HIP.  n = 0 launches nothing.
 */
typedef struct q4gsw_adamw_params {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
} q4gsw_adamw_params;
q4gsw_status q4gsw_adamw_step(float *param, const float *grad, float *exp_avg, float *exp_avg_sq, int64_t n,
                              const q4gsw_adamw_params *hp, int64_t step, void *stream);

/*
 * Embedding row gather: out[t, k] = dequant(W)[ids[t], k], for t < T and k < K.
 * The embedding_q4gsw op of the Gemma 4 ExecuTorch export (maintainer comment on the
 * react-native-executorch issue "Upstream the Gemma 4 Vulkan support we carry on our
 * ExecuTorch fork"), with the table in a linear weight's packed layout (the
 * is_linear_weight flag of the WebGPU pull request that keeps the Q4 embedding's shader
 * controls across resize): the weight packed once for forward, input gradient and QKV
 * serves as the table of N rows of K columns, with no re-pack.
 *   ids  device int64 [T]; an id outside [0, N) gives a row of zeros (the pages leave
 *        this open; it is checked on the device, so it is not an error status)
 *   out  device fp32 [T, K]; must not overlap ids or the packed weight (E_ALIAS)
 * Values are exact for fp16 scales ((code - 8) * scale fits fp32) and the fp32 product,
 * correctly rounded, for fp32 scales.  No workspace.  E_SHAPE for T < 1, T > 2^23, or
 * T * ceil(ceil(K / 8) / 64) >= 2^31.
 */
q4gsw_status q4gsw_embedding(const q4gsw_weight *w, const int64_t *ids, int64_t T, float *out,
                             void *stream);

/* Route attestation: the q4gsw_route_id a plain call (no options) with these
 * arguments takes (Q4GSW_ROUTE_NONE if it would fail validation).  For
 * Q4GSW_OP_QKV pass Wq.  This is the attestation of the WebGPU SDPA routing pull
 * request in the BK64 QKV stack, which reports the route a shape takes so a test
 * harness can tell which kernel served it.  Pure host function. */
int32_t q4gsw_route(int32_t op, const q4gsw_weight *w, int64_t M, int32_t act_dtype);
const char *q4gsw_route_name(int32_t route);

/* Plan attestation for tests and benchmarks: how a call with these arguments and
 * `opts` (NULL: none) runs.  For Q4GSW_OP_QKV pass the three weights (wk, wv are
 * ignored for the other ops and may be NULL).  Host only, no GPU work; the forward
 * plan weighs the resident blocks per CU of the current device.  Returns
 * Q4GSW_E_NULL without `info`, the validation status of the descriptors and of
 * `opts`, else Q4GSW_OK; a call that would fail validation (or that the requested
 * route cannot serve) reports route Q4GSW_ROUTE_NONE. */
typedef struct q4gsw_plan_info {
    int32_t route;          /* as q4gsw_route */
    int32_t tile_rows;      /* rows (M) of the MFMA block tile (forward / QKV: 128 or 64;
                               input gradient: 128); 0 without an MFMA GEMM */
    int32_t splits;         /* contraction splits across blocks (1: none; more: a reduction
                               launch sums the fp32 partials in split order) */
} q4gsw_plan_info;
q4gsw_status q4gsw_plan(int32_t op, const q4gsw_weight *w, const q4gsw_weight *wk, const q4gsw_weight *wv,
                        int64_t M, int32_t act_dtype, const q4gsw_options *opts, q4gsw_plan_info *info);

const char *q4gsw_status_str(int32_t status);

/* Layout version and a build identifier string. */
uint32_t q4gsw_layout_version(void);
const char *q4gsw_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4GSW_H */
