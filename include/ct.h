/*
 * ct.h - C ABI of the transposed-convolution / pooling library (libct.so),
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Operations (each defined on a POPCORNBENCH web page, one problem per page):
 *   [p50] "Kimi-K2.6 l2_p50": ConvTranspose3d -> x scale1 -> AvgPool3d(2) ->
 *         + bias -> x scale2, fused into one kernel that never materialises
 *         the pre-pool tensor.
 *   [p46] "Kimi-K2.6 l1_p46": AvgPool3d(k3, s2, p1) with zero padding counted
 *         in the divisor (count_include_pad, divisor 27).
 *   [p74] "Kimi-K2.6 l1_p74": ConvTranspose1d with dilation (k5, s1, p0, d3 on
 *         the page).
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, contiguous, row-major (NCDHW / NCL).  Weights are
 *     laid out [Cin][Cout][k...] as PyTorch's transposed convolutions store
 *     them.  Output sizes follow PyTorch's formulas (ct_convT_out_len,
 *     ct_pool_out_len).
 *   - Tensor pointers are DEVICE pointers (hipMalloc'd or from any allocator
 *     of the current device).  The caller owns every buffer, allocates the
 *     output, and keeps all buffers alive until the work on `stream` is done.
 *     The library allocates no device memory and keeps no state besides a
 *     per-thread error string and per-device facts it queries once and
 *     caches (compute-unit count, kernel occupancies, granted LDS sizes).
 *   - fp32 pointers must be 4-byte aligned, bf16 pointers 2-byte aligned.
 *     The output must not overlap any input.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; nothing synchronises.  A device fault surfaces at the
 *     caller's next synchronisation, not in the return value.  After the
 *     first call of an operation on a device, a call enqueues nothing but
 *     kernel launches (no allocation, memset or copy), so it may be captured
 *     in a HIP graph on `stream` and replayed.
 *   - Every call returns a ct_status.  All argument checks run before any HIP
 *     call, so a rejected call touches neither the GPU nor the HIP runtime.
 *     ct_last_error() gives a human-readable reason for the last non-OK
 *     status on the calling thread.
 */
#ifndef CT_H
#define CT_H

#include <stdint.h>

#if defined(__GNUC__)
#define CT_API __attribute__((visibility("default")))
#else
#define CT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CT_OK = 0,
    CT_EINVAL = 1,       /* null required pointer, bad size, empty output, misalignment, overlap */
    CT_EUNSUPPORTED = 2, /* well-formed request this library does not implement */
    CT_EHIP = 3          /* the HIP runtime reported an error when launching */
} ct_status;

typedef enum {
    CT_F32 = 0,          /* IEEE binary32 */
    CT_BF16 = 1          /* bfloat16 (upper half of a binary32) */
} ct_dtype;

/*
 * Output length of a transposed convolution along one axis:
 *   (in - 1) * stride - 2 * pad + dilation * (k - 1) + out_pad + 1.
 * [p50], passage deriving the ConvTranspose3d output shape (16/32/32 ->
 * 31/63/63); [p74], opening passage (L_out = L + 12 at k5 d3).
 * Pure host arithmetic, evaluated without overflow; may return a value <= 0
 * for impossible geometry, and returns -1 when the length lies outside int64.
 */
CT_API int64_t ct_convT_out_len(int64_t in, int64_t k, int64_t stride, int64_t pad,
                         int64_t out_pad, int64_t dilation);

/*
 * Output length of an average pool along one axis, floor mode:
 *   floor((in + 2 * pad - k) / stride) + 1.
 * [p50], passage on AvgPool3d(2) (31 -> 15); [p46], opening passage
 * (128 -> 64, 256 -> 128).  Returns <= 0 when no window fits, -1 when the
 * length lies outside int64 (evaluated without overflow).  stride == 0 means
 * stride = k (PyTorch's default).
 */
CT_API int64_t ct_pool_out_len(int64_t in, int64_t k, int64_t stride, int64_t pad);

/*
 * Fused ConvTranspose3d -> x scale1 -> AvgPool3d -> + bias -> x scale2
 * ([p50], problem statement and the model's forward):
 *
 *   Y   = ConvTranspose3d(x, w, stride, pad, out_pad) + conv_bias
 *   out = ((AvgPool3d_{pool_k, pool_s}(Y * scale1)) + bias) * scale2
 *
 * computed directly per pooled voxel from the 2x2x2 input taps each pooled
 * voxel depends on ([p50], passages on the stride-2 parity rule and on
 * grouping the 27 weight terms by input tap); the pre-pool tensor Y is never
 * written.
 *
 *   x          [N, Cin, D, H, W], dtype x_dtype
 *   w          [Cin, Cout, k, k, k], dtype w_dtype
 *   conv_bias  [Cout] fp32, or NULL (= 0)
 *   bias       [Cout] fp32, or NULL (= 0); the page's [Cout,1,1,1] parameter
 *   out        [N, Cout, Dp, Hp, Wp] fp32, with Do = ct_convT_out_len(D, k,
 *              stride, pad, out_pad, 1) and Dp = ct_pool_out_len(Do, pool_k,
 *              pool_s, 0) (likewise H, W).  At k3 s2 p1 with a 2-pool,
 *              Dp = D - 1 for every D ([p50], passage on arbitrary sizes).
 *
 * Geometry: any k >= 1, stride >= 1, pad >= 0, 0 <= out_pad < stride
 * (PyTorch's rule at dilation 1), pool_k >= 1, pool_s >= 1 (0 = pool_k);
 * (x_dtype, w_dtype) = (CT_F32, CT_F32) or (CT_BF16, CT_BF16); accumulation
 * and output are fp32.  Implementations:
 *   - k = 3, stride = 2, pad = 1, pool 2/2 (the page's geometry) with
 *     out_pad 0 or 1 and Cin <= 128: matrix-core kernels that contract the 8
 *     input taps of a pooled voxel with the grouped (summed) filter, taps
 *     past the far edge (out_pad = 1) reading 0.  fp32 runs on an LDS-slab
 *     pipeline (Cin <= 4, large calls) or a direct kernel that loads its taps
 *     from memory.  bf16 with out_pad 0, Cin <= 32, W a multiple of 8 up to
 *     4096 and x 16-byte aligned runs on a bf16 kernel that represents the
 *     summed filter as a bf16 hi + lo pair (the result matches an fp32
 *     computation on the same bf16 inputs to ~2^-17 relative per term),
 *     except Cin <= 4 with Cout <= 16, which, like every other bf16 call at
 *     this geometry, runs on the direct kernel with the taps widened exactly
 *     to fp32.
 *   - the same conv and pool geometry with Cin > 128, when Cin * Cout <=
 *     1024: the same effective-filter sum on the vector ALUs.
 *   - anything else: a general gather kernel on the vector ALUs (one thread
 *     per pooled voxel summing the pool window of transposed-convolution
 *     values), fp32 arithmetic on the (exactly widened) inputs.
 * Mixed dtypes, lengths or Cin/Cout beyond 2^30, or k / pool_k beyond 1024
 * -> CT_EUNSUPPORTED.  An empty output (e.g. D = 1 at the page's geometry)
 * -> CT_EINVAL.
 */
CT_API ct_status ct_convT3d_scale_pool_bias(
    const void *x, int x_dtype,
    const void *w, int w_dtype,
    const float *conv_bias, const float *bias,
    float scale1, float scale2,
    int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W, int64_t Cout,
    int k, int stride, int pad, int out_pad, int pool_k, int pool_s,
    float *out, void *stream);

/*
 * ConvTranspose3d alone, materialising its output ([p50], the model's first
 * layer; the page's estimate of the traffic the fusion saves compares the
 * fused chain with this layer followed by a separate pool):
 *   y[n,co,od,oh,ow] = sum_ci sum_{kd,kh,kw} x[n,ci,id,ih,iw] * w[ci,co,kd,kh,kw]
 *                      (+ bias[co])
 * over the taps with od = id*stride - pad + kd (likewise h, w) inside the
 * output, i.e. id = (od + pad - kd) / stride where that division is exact.
 *
 *   x     [N, Cin, D, H, W], dtype x_dtype
 *   w     [Cin, Cout, k, k, k], dtype w_dtype (== x_dtype)
 *   bias  [Cout] fp32, or NULL (= 0)
 *   out   [N, Cout, Do, Ho, Wo] fp32, Do = ct_convT_out_len(D, k, stride,
 *         pad, out_pad, 1) (likewise H, W)
 *
 * Geometry and limits as for ct_convT3d_scale_pool_bias.  Computed by the
 * general gather kernel (one thread per output), fp32 arithmetic.
 */
CT_API ct_status ct_convT3d(const void *x, int x_dtype,
                     const void *w, int w_dtype,
                     const float *bias,
                     int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W, int64_t Cout,
                     int k, int stride, int pad, int out_pad,
                     float *out, void *stream);

/*
 * AvgPool3d over zero padding ([p46], opening passages):
 *   out[n,c,d,h,w] = (sum over kd,kh,kw < k of x[n,c, d*s - p + kd,
 *                     h*s - p + kh, w*s - p + kw]) / divisor
 * where taps outside the input read as 0.  The divisor is k^3 when
 * count_include_pad = 1 (the page's case: 27 at k = 3) and the number of
 * taps inside the input when count_include_pad = 0 ([p46], passage on the
 * divisor of border windows).
 *
 *   x    [N, C, D, H, W] fp32
 *   out  [N, C, Do, Ho, Wo] fp32, Do = ct_pool_out_len(D, k, stride, pad)
 *
 * Geometry: k >= 1, stride >= 0 (0 = k), 0 <= pad <= k/2 (PyTorch's rule),
 * floor mode.  k = 3, stride 2, pad 1 (either count_include_pad) runs on a
 * streaming kernel that reads each input once (per-slice size below 2^31
 * elements): planes of at most 4096 elements several slices per workgroup
 * through LDS, larger ones as separable row sums; anything else on a
 * general gather kernel (one thread per output; lengths and stride up to
 * 2^30, k up to 1024, else CT_EUNSUPPORTED).
 */
CT_API ct_status ct_avgpool3d(const float *x,
                       int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                       int k, int stride, int pad, int count_include_pad,
                       float *out, void *stream);

/*
 * The same AvgPool3d on bf16 data ([p46]'s operation with the tensor in
 * bf16, as PyTorch's AvgPool3d runs on a bf16 tensor): every tap is widened
 * exactly to fp32, the window sum and the division are fp32, and each mean is
 * rounded to the nearest bf16 (ties to even; NaN stays NaN).
 *
 *   x    [N, C, D, H, W] bf16 bit patterns (uint16_t), 2-byte aligned
 *   out  [N, C, Do, Ho, Wo] bf16 bit patterns, sizes as for ct_avgpool3d
 *
 * Geometry, limits, ownership and errors as for ct_avgpool3d (sizes in
 * bf16 elements).  k = 3, stride 2, pad 1 (either count_include_pad) runs on
 * the same separable streaming kernels (the vector one when W % 4 == 0, x is
 * 8-byte and out 4-byte aligned); anything else on the general gather kernel.
 */
CT_API ct_status ct_avgpool3d_bf16(const uint16_t *x,
                       int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                       int k, int stride, int pad, int count_include_pad,
                       uint16_t *out, void *stream);

/*
 * Transposed 1D convolution ([p74], gather form derived on the page):
 *   y[n,co,o] = sum_ci sum_{k<K} x[n,ci,(o + pad - dilation*k)/stride]
 *               * w[ci,co,k]  (+ bias[co])
 * over the terms whose index is an integer inside [0, L); with stride 1 and
 * pad 0 this is y[n,co,o] = sum_ci sum_k x[n,ci,o - dilation*k] w[ci,co,k].
 * The weights are used unflipped.
 *
 *   x     [N, Cin, L], dtype x_dtype
 *   w     [Cin, Cout, K], dtype w_dtype
 *   bias  [Cout] fp32, or NULL (= 0)
 *   out   [N, Cout, L_out] fp32, L_out = ct_convT_out_len(L, K, stride, pad,
 *         out_pad, dilation)
 *
 * Geometry: K >= 1, stride >= 1, pad >= 0, dilation >= 1,
 * 0 <= out_pad < max(stride, dilation) (PyTorch's rule);
 * (x_dtype, w_dtype) = (CT_F32, CT_F32) or (CT_BF16, CT_BF16).
 *   - fp32, stride 1, pad 0, out_pad 0 (the page's case): an implicit GEMM
 *     on the fp32 matrix cores (full fp32 products and accumulation), as
 *     long as the weights (64 * K * Cin4 floats, Cin4 = Cin rounded up to a
 *     multiple of 4) and one input strip (Cin4 rows of 256 +
 *     dilation*(K-1) floats, padded) fit the 160 KiB LDS of one gfx950
 *     workgroup (Cin=32, K=5, dilation 3 needs 74 KiB).
 *   - fp32 at the page's channels and taps (Cin 32, K 5, dilation 3, L a
 *     multiple of 4, x 16-byte aligned): stride 1 with any pad and output
 *     padding on the same matrix-core kernel over a shifted output window
 *     (any L_out: when L_out % 4 != 0 or out is not 16-byte aligned, rows
 *     are stored with 4-byte aligned vectors); stride 2 to 8 with any
 *     pad and output padding as stride-1 gathers over the residue classes of
 *     o + pad on the fp32 matrix cores (a class without taps, such as
 *     classes 1 and 2 at dilation 3 and stride 3, outputs the bias).
 *   - bf16 at the page's channels and taps (Cin 32, K 5, dilation 3), stride
 *     1 with any pad and output padding, L a multiple of 8, x 16-byte
 *     aligned: an implicit GEMM on the bf16 matrix cores with fp32
 *     accumulation (a pad shifts the output window; any L_out and 4-byte
 *     aligned out).
 *   - anything else: a general gather kernel (one thread per output), fp32
 *     arithmetic on the exactly widened inputs; lengths, Cin, Cout, pad and
 *     dilation*(K-1) up to 2^30, else CT_EUNSUPPORTED.
 */
CT_API ct_status ct_convT1d(const void *x, int x_dtype,
                     const void *w, int w_dtype,
                     const float *bias,
                     int64_t N, int64_t Cin, int64_t L, int64_t Cout,
                     int K, int stride, int pad, int dilation, int out_pad,
                     float *out, void *stream);

/* Static name of a status code ("CT_OK", ...). */
CT_API const char *ct_status_str(int status);

/* Reason for the last non-OK status returned on this thread ("" if none). */
CT_API const char *ct_last_error(void);

/* Library version string. */
CT_API const char *ct_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CT_H */
